"""GPU parity at the edges of the C ABI, against the CPU fp64 oracle: the
largest visit count one call accepts, empty and one-key blocks, MHA decode
(G = 1), wide groups (G = 16) and multi-query attention (G = 64, also in the
fan-out decode), strided views out of fused QKV buffers,
head-major layouts, an explicit logit scale, every split mode, and two
calls running at once on two streams.  Every case prints its name,
shape and seed before it touches the GPU."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_blockwise_long_amd import blockattn as ba
from exact_blockwise_long_amd import synth
from oracle import attention as ora
from tests import helpers as H

pytestmark = pytest.mark.gpu

MAX_VISITS = 32   # BLOCKATTN_MAX_VISITS


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ba.load()
    yield
    torch.cuda.synchronize()


def run_and_check(q, k, v, lens, order, *, Hkv, q_pos0, causal, split_mode, scale=0.0, qd=None, kd=None, vd=None,
                  what="", kpos0=0):
    """fwd_block over blocks cut from k, v in the given lengths (keys at
    positions kpos0, kpos0 + 1, ... in block order), then finalize; compared
    with the oracle's attention."""
    T, Hq, D = q.shape
    qd = H.to_device(q) if qd is None else qd
    kd = H.to_device(k) if kd is None else kd
    vd = H.to_device(v) if vd is None else vd
    blocks, off = [], 0
    for n in lens:
        blocks.append((kd[off:off + n], vd[off:off + n], kpos0 + off))
        off += n
    st = ba.new_state(T * Hq, D)
    ba.fwd_block(qd, blocks, order, st, reset=True, n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal,
                 split_mode=split_mode, scale=scale)
    out, lse = ba.finalize(st)
    torch.cuda.synchronize()
    s = scale if scale > 0 else 1.0 / np.sqrt(D)
    a_ref, _, _, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), s, q_pos0 + np.arange(T),
                                      kpos0 + np.arange(k.shape[0]), causal)
    stats = H.assert_bf16_out(H.host(out).reshape(T, Hq, D), a_ref, what)
    H.assert_close(H.host(lse).reshape(T, Hq), lse_ref, H.BF16_LSE, what + " lse")
    print(f"    {what}: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}", flush=True)
    return out, lse


@pytest.mark.parametrize("split_mode", [0, 1, 2])
def test_max_visits_in_one_call(split_mode):
    """32 blocks in one call, in a shuffled order: empty, one-key, ragged and
    multi-tile blocks; causal with the queries in the middle of the keys, so
    later blocks are partly or wholly in the future."""
    seed, T, Hq, Hkv, D = 81, 40, 8, 2, 128
    lens = [[1, 0, 63, 64, 65, 7, 128, 200][i % 8] for i in range(MAX_VISITS)]
    order = synth.rng(seed + 1).permutation(MAX_VISITS).tolist()
    L = sum(lens)
    q_pos0 = L // 2
    announce(f"max visits: {MAX_VISITS} blocks, {L} keys, T={T} q_pos0={q_pos0} split_mode={split_mode} seed {seed}")
    g = synth.rng(seed)
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    run_and_check(q, k, v, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=True, split_mode=split_mode,
                  what=f"{MAX_VISITS} visits mode {split_mode}")


@pytest.mark.parametrize("split_mode", [0, 1, 2])
def test_positions_beyond_32_bits(split_mode):
    """A causal walk whose absolute positions start at 3e9 (past 2^31): the
    queries sit inside the keys, so blocks are wholly visible, straddle the
    diagonal or lie wholly in the future."""
    seed, T, Hq, Hkv, D, lens = 84, 150, 8, 2, 128, [200, 65, 300, 129]
    base = 3_000_000_000
    L = sum(lens)
    q_pos0 = base + 260
    announce(f"positions past 2^31: keys at {base}..{base + L - 1}, q_pos0={q_pos0}, T={T}, mode {split_mode}, "
             f"seed {seed}")
    g = synth.rng(seed)
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    run_and_check(q, k, v, lens, [3, 1, 0, 2], Hkv=Hkv, q_pos0=q_pos0, causal=True, split_mode=split_mode,
                  kpos0=base, what=f"positions past 2^31 mode {split_mode}")


@pytest.mark.parametrize("Hq,Hkv,T,causal", [(8, 8, 1, False), (8, 8, 1, True), (16, 1, 33, True),
                                             (16, 1, 33, False), (64, 1, 33, True), (64, 1, 1, False)])
def test_group_sizes_and_decode(Hq, Hkv, T, causal):
    """MHA (G = 1) with a single query token, a 16-wide group, and multi-query
    attention (64 query heads on one KV head: several row tiles per token
    block, the wide workgroups)."""
    seed, D, lens = 82, 128, [300, 1, 129]
    announce(f"groups: Hq={Hq} Hkv={Hkv} T={T} causal={causal} lens={lens} seed {seed}")
    g = synth.rng(seed)
    L = sum(lens)
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    for mode in (0, 1, 2):
        run_and_check(q, k, v, lens, [2, 0, 1], Hkv=Hkv, q_pos0=L - T, causal=causal, split_mode=mode,
                      what=f"G={Hq // Hkv} T={T} mode {mode}")


@pytest.mark.parametrize("nb", [16, 1])
def test_fanout_multi_query(nb):
    """Fan-out decode with 64 query heads on one KV head: 64 rows per branch,
    so 16 branches make one KV head's 1024 rows (the wide launch)."""
    seed, Hq, Hkv, D, P, S = 83, 64, 1, 128, 3000, 257
    announce(f"fanout multi-query: nb={nb} Hq={Hq} Hkv={Hkv} D={D} P={P} S={S} seed {seed}")
    g = synth.rng(seed)
    q = synth.normal(g, (nb, Hq, D), 0.5, "bf16")
    pk = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    pv = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    sk = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    sv = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    out, lse = ba.fanout_prefix_decode(*(H.to_device(t) for t in (q, pk, pv, sk, sv)))
    torch.cuda.synchronize()
    a_ref, lse_ref = ora.fanout_decode(q.f64(), pk.f64(), pv.f64(), sk.f64(), sv.f64(), 1.0 / np.sqrt(D))
    stats = H.assert_bf16_out(H.host(out), a_ref, f"fanout multi-query nb={nb}")
    H.assert_close(H.host(lse), lse_ref, H.BF16_LSE, "lse")
    print(f"    max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}", flush=True)


def test_strided_views_and_explicit_scale():
    """Q, K and V as views into fused buffers ([T, 3, Hq, D] and [L, 2, Hkv, D]:
    token strides of 3*Hq*D and 2*Hkv*D elements), with an explicit logit
    scale; the backward with dO a view of the same strides."""
    seed, T, Hq, Hkv, D, lens, scale = 83, 70, 8, 2, 64, [100, 37], 0.07
    announce(f"strided views: q from [T,3,Hq,D], k/v from [L,2,Hkv,D], D={D} scale={scale} seed {seed}")
    g = synth.rng(seed)
    L = sum(lens)
    qkv = synth.normal(g, (T, 3, Hq, D), 0.5, "bf16")
    kv = synth.normal(g, (L, 2, Hkv, D), 0.5, "bf16")
    q = synth.Tensor(np.ascontiguousarray(qkv.storage[:, 0]), "bf16")
    k = synth.Tensor(np.ascontiguousarray(kv.storage[:, 0]), "bf16")
    v = synth.Tensor(np.ascontiguousarray(kv.storage[:, 1]), "bf16")
    qkvd, kvd = H.to_device(qkv), H.to_device(kv)
    qd, kd, vd = qkvd[:, 0], kvd[:, 0], kvd[:, 1]
    assert qd.stride(0) == 3 * Hq * D and kd.stride(0) == 2 * Hkv * D
    for causal in (False, True):
        for mode in (1, 2):
            run_and_check(q, k, v, lens, [1, 0], Hkv=Hkv, q_pos0=L - T, causal=causal, split_mode=mode, scale=scale,
                          qd=qd, kd=kd, vd=vd, what=f"strided causal={causal} mode {mode}")
    # backward through the same views: dO is the third slot of the fused buffer
    dod = qkvd[:, 2]
    do = synth.Tensor(np.ascontiguousarray(qkv.storage[:, 2]), "bf16")
    blocks = [(kd[:lens[0]], vd[:lens[0]], 0), (kd[lens[0]:], vd[lens[0]:], lens[0])]
    st = ba.new_state(T * Hq, D)
    ba.fwd_block(qd, blocks, [1, 0], st, reset=True, n_kv_heads=Hkv, q_pos0=L - T, causal=True, scale=scale)
    out, lse = ba.finalize(st)
    delta = ba.bwd_delta(out, dod.reshape(T * Hq, D) if dod.is_contiguous() else dod.contiguous().reshape(T * Hq, D))
    dq = torch.zeros(T * Hq, D, dtype=torch.float32, device="cuda")
    dkv = [(torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda"),
            torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda")) for n in lens]
    ba.bwd_block(qd, dod, lse, delta, blocks, [1, 0], dq, dkv, n_kv_heads=Hkv, q_pos0=L - T, causal=True, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = ora.attention_grads(q.f64(), k.f64(), v.f64(), do.f64(), scale, L - T + np.arange(T), None, True)
    for got, ref, name in ((H.host(dq).reshape(T, Hq, D), rq, "dQ"),
                           (np.concatenate([H.host(a) for a, _ in dkv]), rk, "dK"),
                           (np.concatenate([H.host(b) for _, b in dkv]), rv, "dV")):
        err = np.abs(got - ref)
        mx, mn = err.max() / np.abs(ref).max(), err.mean() / np.abs(ref).mean()
        print(f"    strided backward {name}: {mx:.2e} / {mn:.2e}", flush=True)
        assert mx <= 2e-2 and mn <= 5e-3, f"strided backward {name}"


def test_head_major_layouts():
    """Q stored as [Hq, T, D] and K, V as [Hkv, L, D], passed as [T, Hq, D] and
    [L, Hkv, D] views (token stride D, head stride T*D or L*D): both forward
    paths, the fused forward-and-finalise call, and the backward with dO in
    the same layout as Q."""
    seed, T, Hq, Hkv, D, lens, q_pos0 = 84, 150, 8, 2, 128, [130, 64], 60
    announce(f"head-major layouts T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} q_pos0={q_pos0} seed {seed}")
    g = synth.rng(seed)
    L = sum(lens)
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    do = synth.normal(g, (T, Hq, D), 0.5, "bf16")

    def head_major(t):
        return H.to_device(t).permute(1, 0, 2).contiguous().permute(1, 0, 2)

    qd, kd, vd, dod = head_major(q), head_major(k), head_major(v), head_major(do)
    assert qd.stride() == (D, T * D, 1) and kd.stride() == (D, L * D, 1)
    for mode in (1, 2):
        run_and_check(q, k, v, lens, [1, 0], Hkv=Hkv, q_pos0=q_pos0, causal=True, split_mode=mode, qd=qd, kd=kd,
                      vd=vd, what=f"head-major mode {mode}")
    blocks = [(kd[:lens[0]], vd[:lens[0]], 0), (kd[lens[0]:], vd[lens[0]:], lens[0])]
    st = ba.new_state(T * Hq, D)
    out, lse = ba.fwd_block_finalize(qd, blocks, [1, 0], st, reset=True, n_kv_heads=Hkv, q_pos0=q_pos0, causal=True)
    torch.cuda.synchronize()
    a_ref, _, _, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), 1.0 / np.sqrt(D), q_pos0 + np.arange(T), None, True)
    H.assert_bf16_out(H.host(out).reshape(T, Hq, D), a_ref, "head-major fused")
    H.assert_close(H.host(lse).reshape(T, Hq), lse_ref, H.BF16_LSE, "head-major fused lse")
    delta = ba.bwd_delta(out, dod.contiguous().reshape(T * Hq, D))
    dq = torch.zeros(T * Hq, D, dtype=torch.float32, device="cuda")
    dkv = [(torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda"),
            torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda")) for n in lens]
    ba.bwd_block(qd, dod, lse, delta, blocks, [1, 0], dq, dkv, n_kv_heads=Hkv, q_pos0=q_pos0, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = ora.attention_grads(q.f64(), k.f64(), v.f64(), do.f64(), 1.0 / np.sqrt(D), q_pos0 + np.arange(T),
                                     None, True)
    for got, ref, name in ((H.host(dq).reshape(T, Hq, D), rq, "dQ"),
                           (np.concatenate([H.host(a) for a, _ in dkv]), rk, "dK"),
                           (np.concatenate([H.host(b) for _, b in dkv]), rv, "dV")):
        err = np.abs(got - ref)
        mx, mn = err.max() / np.abs(ref).max(), err.mean() / np.abs(ref).mean()
        print(f"    head-major backward {name}: {mx:.2e} / {mn:.2e}", flush=True)
        assert mx <= 2e-2 and mn <= 5e-3, f"head-major backward {name}"


def test_two_streams_at_once():
    """Work goes on the caller's stream and the library keeps no state of its
    own: a split forward-and-finalise call and a fan-out decode issued three
    times each on two side streams (default priority) run concurrently and both
    match the oracle."""
    seed = 85
    announce(f"two streams at once: fwd_block_finalize (split) and fanout_prefix_decode, seed {seed}")
    g = synth.rng(seed)
    T, Hq, Hkv, D, lens, q_pos0 = 300, 8, 2, 128, [200, 77, 129, 64], 350
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (sum(lens), Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (sum(lens), Hkv, D), 0.5, "bf16")
    nb, P, S = 4, 1000, 37
    fq = synth.normal(g, (nb, Hq, D), 0.5, "bf16")
    pk = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    pv = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    sk = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    sv = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks, off = [], 0
    for n in lens:
        blocks.append((kd[off:off + n], vd[off:off + n], off))
        off += n
    fdev = [H.to_device(t) for t in (fq, pk, pv, sk, sv)]
    # every buffer is allocated before the side streams start
    kw = dict(n_kv_heads=Hkv, q_pos0=q_pos0, causal=True, split_mode=2)
    st = ba.new_state(T * Hq, D)
    out_a = torch.empty(T * Hq, D, dtype=torch.bfloat16, device="cuda")
    lse_a = torch.empty(T * Hq, dtype=torch.float32, device="cuda")
    ws_a = torch.empty(max(1, ba.fwd_workspace_bytes(qd, blocks, [2, 0, 3, 1], **kw)), dtype=torch.uint8,
                       device="cuda").fill_(0xFF)
    out_b = torch.empty(nb, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse_b = torch.empty(nb, Hq, dtype=torch.float32, device="cuda")
    ws_b = torch.empty(ba.fanout_workspace_bytes(nb, Hq, Hkv, D, P, S), dtype=torch.uint8, device="cuda").fill_(0xFF)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            ba.fwd_block_finalize(qd, blocks, [2, 0, 3, 1], st, reset=True, out=out_a, lse=lse_a, workspace=ws_a,
                                  **kw)
        with torch.cuda.stream(s2):
            ba.fanout_prefix_decode(*fdev, workspace=ws_b, out=out_b, lse=lse_b)
    torch.cuda.synchronize()
    a_ref, _, _, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), 1.0 / np.sqrt(D), q_pos0 + np.arange(T), None, True)
    H.assert_bf16_out(H.host(out_a).reshape(T, Hq, D), a_ref, "stream 1 forward")
    H.assert_close(H.host(lse_a).reshape(T, Hq), lse_ref, H.BF16_LSE, "stream 1 lse")
    b_ref, lse_b_ref = ora.fanout_decode(fq.f64(), pk.f64(), pv.f64(), sk.f64(), sv.f64(), 1.0 / np.sqrt(D))
    H.assert_bf16_out(H.host(out_b), b_ref, "stream 2 fan-out")
    H.assert_close(H.host(lse_b), lse_b_ref, H.BF16_LSE, "stream 2 lse")
