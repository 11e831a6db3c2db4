"""GPU parity of the blockwise backward (through the C ABI) against the CPU
fp64 oracle's attention gradients.

The forward runs on the GPU (fwd_block + finalize), its bf16 output and
log-sum-exp feed bwd_delta and bwd_block, and dQ, dK, dV are compared with
the oracle's exact gradients of the same bf16 inputs.  Every case prints its
name, shape and seed before it touches the GPU.

Tolerance (a reading: no gradient tolerance is fixed for the method).  The
kernels round P and dS to bf16 for the matrix cores and read the forward's
bf16 output for D = rowsum(dO * A); each of those is a relative 2^-9
perturbation of a term of a sum of hundreds of terms with random signs.  The
errors are judged against the gradient's own scale: the largest error at most
2e-2 of the largest reference magnitude, the mean error at most 5e-3 of the
mean reference magnitude.
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

MAX_REL, MEAN_REL = 2e-2, 5e-3


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ba.load()
    yield
    torch.cuda.synchronize()


def check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    scale_max = float(np.abs(ref).max()) if ref.size else 0.0
    scale_mean = float(np.abs(ref).mean()) if ref.size else 0.0
    mx = float(err.max()) / max(scale_max, 1e-30) if err.size else 0.0
    mn = float(err.mean()) / max(scale_mean, 1e-30) if err.size else 0.0
    print(f"    {what}: max err / max|ref| {mx:.2e}, mean err / mean|ref| {mn:.2e} "
          f"(max|ref| {scale_max:.3e})", flush=True)
    assert mx <= MAX_REL and mn <= MEAN_REL, f"{what}: relative errors {mx:.3e} / {mn:.3e}"


def make_case(seed, T, Hq, Hkv, D, lens):
    g = synth.rng(seed)
    L = sum(lens)
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    do = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    return q, k, v, do


def device_blocks(kd, vd, lens, kpos0=0):
    blocks, off = [], 0
    for n in lens:
        blocks.append((kd[off:off + n], vd[off:off + n], kpos0 + off))
        off += n
    return blocks


def gpu_grads(q, k, v, do, lens, order, *, Hkv, q_pos0, causal, per_visit, kpos0=0):
    """Forward on the GPU, then the backward over the same visits (reversed
    and one call per visit when ``per_visit``, as a ring's backward runs).
    The keys sit at positions kpos0, kpos0 + 1, ... in block order."""
    T, Hq, D = q.shape
    qd, kd, vd, dod = (H.to_device(x) for x in (q, k, v, do))
    blocks = device_blocks(kd, vd, lens, kpos0)
    st = ba.new_state(T * Hq, D)
    ba.fwd_block(qd, blocks, order, st, reset=True, n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal, split_mode=1)
    out, lse = ba.finalize(st)
    delta = ba.bwd_delta(out, dod)
    dq = torch.zeros(T * Hq, D, dtype=torch.float32, device="cuda")
    dkv = [(torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda"),
            torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda")) for n in lens]
    if per_visit:
        for j in reversed(order):
            ba.bwd_block(qd, dod, lse, delta, blocks, [j], dq, dkv, n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal)
    else:
        ba.bwd_block(qd, dod, lse, delta, blocks, order, dq, dkv, n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal)
    torch.cuda.synchronize()
    dk = torch.cat([x[0] for x in dkv], 0)
    dv = torch.cat([x[1] for x in dkv], 0)
    return H.host(dq).reshape(T, Hq, D), H.host(dk), H.host(dv)


def oracle_grads(q, k, v, do, q_pos0, causal, kpos0=0):
    T, _, D = q.shape
    L = k.shape[0]
    return ora.attention_grads(q.f64(), k.f64(), v.f64(), do.f64(), 1.0 / np.sqrt(D), q_pos0 + np.arange(T),
                               kpos0 + np.arange(L), causal)


CASES = [
    # (seed, T, Hq, Hkv, D, lens, order, q_pos0, causal): several row and key
    # tiles, ragged tails, GQA, causal diagonals inside tiles, fully future keys.
    (41, 300, 8, 2, 128, [200, 77, 129, 64], [2, 0, 3, 1], 350, True),
    (42, 300, 8, 2, 128, [200, 77, 129, 64], [3, 2, 1, 0], 0, False),
    (43, 130, 4, 4, 64, [65, 128, 31], [1, 2, 0], 150, True),
    (44, 17, 16, 1, 128, [513, 1000], [1, 0], 1400, True),
]


@pytest.mark.parametrize("per_visit", [False, True], ids=["one_call", "per_visit"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_backward_matches_oracle(case, per_visit):
    seed, T, Hq, Hkv, D, lens, order, q_pos0, causal = case
    announce(f"bwd seed {seed} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} order={order} q_pos0={q_pos0} "
             f"causal={causal} per_visit={per_visit}")
    q, k, v, do = make_case(seed, T, Hq, Hkv, D, lens)
    dq, dk, dv = gpu_grads(q, k, v, do, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=causal, per_visit=per_visit)
    rq, rk, rv = oracle_grads(q, k, v, do, q_pos0, causal)
    check_grad(dq, rq, f"seed{seed} dQ")
    check_grad(dk, rk, f"seed{seed} dK")
    check_grad(dv, rv, f"seed{seed} dV")
    if causal:
        # keys after every query's position receive no gradient at all
        L = k.shape[0]
        dead = np.arange(L) > q_pos0 + T - 1
        if dead.any():
            assert not dk[dead].any() and not dv[dead].any(), "gradient on keys no query sees"


# Key counts at the edges of the dK/dV workgroup (128 keys: four pairs of waves
# on 32 keys each, in two 16-key blocks): a pair wholly past a block's end, a
# block ending inside a pair or inside a 16-key block, one key past a
# workgroup; with group sizes that do not divide the 64-row tile (each tile's
# row offsets computed in full) and ones that do (offsets stepped per tile).
EDGE_CASES = [
    # (seed, T, Hq, Hkv, D, lens, q_pos0, causal)
    (48, 65, 6, 2, 128, [31, 33, 96], 80, True),      # G = 3
    (49, 40, 10, 2, 64, [127, 129], 0, False),        # G = 5
    (50, 33, 16, 1, 128, [255, 257], 300, True),      # G = 16
    (51, 129, 8, 1, 128, [32, 128, 1], 140, True),    # G = 8
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=lambda c: f"seed{c[0]}")
def test_backward_dkdv_workgroup_edges(case):
    seed, T, Hq, Hkv, D, lens, q_pos0, causal = case
    order = list(range(len(lens)))[::-1]
    announce(f"bwd workgroup edges seed {seed} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} q_pos0={q_pos0} "
             f"causal={causal}")
    q, k, v, do = make_case(seed, T, Hq, Hkv, D, lens)
    dq, dk, dv = gpu_grads(q, k, v, do, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=causal, per_visit=True)
    rq, rk, rv = oracle_grads(q, k, v, do, q_pos0, causal)
    check_grad(dq, rq, f"seed{seed} dQ")
    check_grad(dk, rk, f"seed{seed} dK")
    check_grad(dv, rv, f"seed{seed} dV")


def test_backward_positions_beyond_32_bits():
    """The backward of a causal walk whose absolute positions start at 3e9."""
    seed, T, Hq, Hkv, D, lens, order = 47, 90, 8, 2, 128, [100, 64, 129], [2, 0, 1]
    base = 3_000_000_000
    q_pos0 = base + 120
    announce(f"bwd positions past 2^31: keys at {base}.., q_pos0={q_pos0}, T={T}, lens={lens}, seed {seed}")
    q, k, v, do = make_case(seed, T, Hq, Hkv, D, lens)
    dq, dk, dv = gpu_grads(q, k, v, do, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=True, per_visit=True,
                           kpos0=base)
    rq, rk, rv = oracle_grads(q, k, v, do, q_pos0, True, kpos0=base)
    check_grad(dq, rq, "dQ")
    check_grad(dk, rk, "dK")
    check_grad(dv, rv, "dV")


def test_backward_single_key_closed_form():
    """One visible key: every row's softmax weight on it is 1, so dP equals D
    row by row, dS = P (dP - D) = 0, and dQ = dK = 0 while dV is the sum of dO
    over the rows.  The GPU's dP and D are two fp32 sums rounded differently,
    so dQ and dK come out at rounding level, not exactly 0."""
    seed, T, Hq, Hkv, D = 48, 65, 16, 2, 128
    lens = [0, 1]
    announce(f"bwd single key: T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} seed {seed}")
    q, k, v, do = make_case(seed, T, Hq, Hkv, D, lens)
    dq, dk, dv = gpu_grads(q, k, v, do, lens, [1, 0], Hkv=Hkv, q_pos0=0, causal=True, per_visit=False)
    g = do.f64().reshape(T, Hkv, Hq // Hkv, D)
    dv_ref = g.sum(axis=(0, 2))[None]                       # [1, Hkv, D]
    print(f"    max |dQ| {np.abs(dq).max():.2e}, max |dK| {np.abs(dk).max():.2e}, "
          f"max |dV - sum dO| {np.abs(dv - dv_ref).max():.2e}", flush=True)
    assert np.abs(dq).max() <= 1e-5 and np.abs(dk).max() <= 1e-5
    assert np.abs(dv - dv_ref).max() <= 1e-4 * max(1.0, np.abs(dv_ref).max())


def test_backward_deterministic():
    seed, T, Hq, Hkv, D, lens, order, q_pos0, causal = CASES[0]
    announce(f"bwd determinism seed {seed}")
    q, k, v, do = make_case(seed, T, Hq, Hkv, D, lens)
    a = gpu_grads(q, k, v, do, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=causal, per_visit=False)
    b = gpu_grads(q, k, v, do, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=causal, per_visit=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_delta_is_rowsum_of_dout_times_out(out_dtype):
    rows, D, seed = 1000, 128, 45
    announce(f"bwd_delta rows={rows} D={D} out={out_dtype} seed {seed}")
    g = synth.rng(seed)
    out = synth.normal(g, (rows, D), 1.0, out_dtype)
    do = synth.normal(g, (rows, D), 1.0, "bf16")
    got = H.host(ba.bwd_delta(H.to_device(out), H.to_device(do)))
    terms = out.f64() * do.f64()
    ref = terms.sum(axis=1)
    bound = 1e-5 * np.abs(terms).sum(axis=1)
    assert np.all(np.abs(got - ref) <= bound), f"worst {np.max(np.abs(got - ref) / bound):.3e} of the bound"


def test_backward_rows_that_see_no_key():
    """Causal rows before every key: the forward leaves them empty (L = -inf)
    and the backward must give them exactly zero dQ and add nothing to any dK,
    dV, with no NaN from exp2(+inf) leaking through the mask."""
    seed, T, Hq, Hkv, D, lens, order, kpos0 = 46, 70, 4, 2, 128, [50, 64], [1, 0], 20
    announce(f"bwd rows without keys seed {seed} T={T} keys at {kpos0}..{kpos0 + sum(lens) - 1} q_pos0=0")
    q, k, v, do = make_case(seed, T, Hq, Hkv, D, lens)
    dq, dk, dv = gpu_grads(q, k, v, do, lens, order, Hkv=Hkv, q_pos0=0, causal=True, per_visit=False, kpos0=kpos0)
    rq, rk, rv = oracle_grads(q, k, v, do, 0, True, kpos0)
    assert not dq[:kpos0].any(), "rows that see no key got a gradient"
    check_grad(dq, rq, f"seed{seed} dQ")
    check_grad(dk, rk, f"seed{seed} dK")
    check_grad(dv, rv, f"seed{seed} dV")
