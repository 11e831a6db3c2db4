"""GPU parity of blockattn_fwd_block_finalize (the last visits of a query
block and its finalisation in one call) against the CPU fp64 oracle, and
against the same visits through blockattn_fwd_block followed by
blockattn_finalize.

The bf16 walk writes A = O / l and LSE = m + ln l from its registers; the
split path finalises in its merge; fp32 problems run the two steps.  Cases
cover both bf16 paths, a state carried in from earlier calls, fp32 output,
an fp32 problem, rows that see no key, and a call with no visits that only
finalises the carried state.  Every case prints its name, shape and seed
before it touches the GPU.
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


def make_case(seed, T, Hq, Hkv, D, lens, dtype):
    g = synth.rng(seed)
    L = sum(lens)
    q = synth.normal(g, (T, Hq, D), 0.5, dtype)
    k = synth.normal(g, (L, Hkv, D), 0.5, dtype)
    v = synth.normal(g, (L, Hkv, D), 0.5, dtype)
    return q, k, v


def device_blocks(kd, vd, lens, kpos0):
    blocks, off = [], 0
    for n in lens:
        blocks.append((kd[off:off + n], vd[off:off + n], kpos0 + off))
        off += n
    return blocks


# (seed, T, Hq, Hkv, D, lens, order, q_pos0, kpos0, causal, split_mode, n_before, dtype, out_dtype):
# the first n_before visits go through fwd_block (state carried), the rest through
# the fused call.  split_mode 1 forces the walk, 2 the key split.
CASES = [
    (71, 300, 8, 2, 128, [200, 77, 129, 64], [2, 0, 3, 1], 350, 0, True, 1, 0, "bf16", "bf16"),
    (72, 300, 8, 2, 128, [200, 77, 129, 64], [3, 2, 1, 0], 0, 0, False, 1, 2, "bf16", "bf16"),
    (73, 130, 4, 4, 64, [65, 128, 31], [1, 2, 0], 150, 0, True, 2, 1, "bf16", "bf16"),
    (74, 130, 4, 4, 64, [65, 128, 31], [1, 2, 0], 150, 0, True, 2, 0, "bf16", "f32"),
    (75, 300, 8, 2, 128, [200, 77], [1, 0], 100, 0, True, 1, 0, "bf16", "f32"),
    (76, 70, 4, 2, 128, [33, 64, 50], [2, 0, 1], 0, 0, True, 0, 1, "f32", "f32"),
    # causal rows at positions 0..19 see no key (keys start at position 20)
    (77, 70, 4, 2, 128, [50, 64], [1, 0], 0, 20, True, 1, 0, "bf16", "bf16"),
    (78, 70, 4, 2, 128, [50, 64], [1, 0], 0, 20, True, 2, 1, "bf16", "bf16"),
]


def ids(c):
    return f"seed{c[0]}_{'walk' if c[10] == 1 else 'split' if c[10] == 2 else 'auto'}_{c[12]}_out{c[13]}"


def run_both(q, k, v, lens, order, *, Hkv, q_pos0, kpos0, causal, split_mode, n_before, out_dtype):
    """The fused call after n_before visits of fwd_block, and the same visits as
    fwd_block + finalize; returns host (out, lse) of both."""
    T, Hq, D = q.shape
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks = device_blocks(kd, vd, lens, kpos0)
    tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    kw = dict(n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal, split_mode=split_mode)
    results = []
    for fused in (True, False):
        st = ba.new_state(T * Hq, D)
        if n_before:
            ba.fwd_block(qd, blocks, order[:n_before], st, reset=True, **kw)
        rest = order[n_before:]
        if fused:
            out, lse = ba.fwd_block_finalize(qd, blocks, rest, st, reset=(n_before == 0), out_dtype=tdt, **kw)
        else:
            ba.fwd_block(qd, blocks, rest, st, reset=(n_before == 0), **kw)
            out, lse = ba.finalize(st, tdt)
        torch.cuda.synchronize()
        results.append((H.host(out).reshape(T, Hq, D), H.host(lse).reshape(T, Hq)))
    return results


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_fused_finalize_matches_oracle(case):
    seed, T, Hq, Hkv, D, lens, order, q_pos0, kpos0, causal, split_mode, n_before, dtype, out_dtype = case
    announce(f"fwd_block_finalize seed {seed} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} order={order} "
             f"q_pos0={q_pos0} kpos0={kpos0} causal={causal} split_mode={split_mode} n_before={n_before} "
             f"{dtype} -> {out_dtype}")
    q, k, v = make_case(seed, T, Hq, Hkv, D, lens, dtype)
    (a_f, lse_f), (a_s, lse_s) = run_both(q, k, v, lens, order, Hkv=Hkv, q_pos0=q_pos0, kpos0=kpos0, causal=causal,
                                          split_mode=split_mode, n_before=n_before, out_dtype=out_dtype)
    L = sum(lens)
    a_ref, _, _, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), 1.0 / np.sqrt(D), q_pos0 + np.arange(T),
                                      kpos0 + np.arange(L), causal)
    if dtype == "bf16":
        H.assert_bf16_out(a_f, a_ref, "fused out")
        H.assert_close(lse_f, lse_ref, H.BF16_LSE, "fused lse")
    else:
        H.assert_close(a_f, a_ref, H.F32_TOL, "fused out")
        H.assert_close(lse_f, lse_ref, H.F32_TOL, "fused lse")
    # Against the two-call path: the same arithmetic up to the final division
    # and the log's argument, so within one rounding of the output type.
    ulp = 2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -22
    scale_a = np.maximum(np.abs(a_s), 1e-3)
    worst = float(np.max(np.abs(a_f - a_s) / scale_a)) if a_s.size else 0.0
    print(f"    fused vs two calls: worst relative out difference {worst:.2e}", flush=True)
    assert worst <= 2 * ulp + 1e-6, f"fused and two-call outputs differ by {worst:.3e} relative"
    H.assert_close(lse_f, lse_s, 1e-5, "fused vs two-call lse")
    empty = np.isneginf(lse_ref)
    if empty.any():
        assert np.all(np.isneginf(lse_f[empty])), "rows without keys must have lse = -inf"
        assert not a_f[empty].any(), "rows without keys must be 0"


def test_fused_finalize_with_no_visits_finalises_the_state():
    """n_visit = 0, reset off: the call only finalises the carried state."""
    seed, T, Hq, Hkv, D, lens = 79, 200, 8, 2, 128, [150, 90]
    announce(f"fwd_block_finalize with no visits seed {seed} T={T} lens={lens}")
    q, k, v = make_case(seed, T, Hq, Hkv, D, lens, "bf16")
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks = device_blocks(kd, vd, lens, 0)
    kw = dict(n_kv_heads=Hkv, q_pos0=100, causal=True, split_mode=1)
    st = ba.new_state(T * Hq, D)
    ba.fwd_block(qd, blocks, [1, 0], st, reset=True, **kw)
    ref_out, ref_lse = ba.finalize(st, torch.bfloat16)
    out, lse = ba.fwd_block_finalize(qd, blocks, [], st, reset=False, **kw)
    torch.cuda.synchronize()
    a_f, a_s = H.host(out), H.host(ref_out)
    worst = float(np.max(np.abs(a_f - a_s) / np.maximum(np.abs(a_s), 1e-3)))
    assert worst <= 2 * 2.0 ** -8 + 1e-6, worst
    H.assert_close(H.host(lse), H.host(ref_lse), 1e-5, "lse")


def test_fused_finalize_with_reset_and_no_keys_gives_empty_rows():
    seed, T, Hq, Hkv, D = 80, 40, 4, 2, 64
    announce(f"fwd_block_finalize reset, no visits seed {seed} T={T}")
    q, k, v = make_case(seed, T, Hq, Hkv, D, [64], "bf16")
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks = device_blocks(kd, vd, [64], 0)
    for split_mode in (1, 2):
        st = ba.new_state(T * Hq, D)
        out, lse = ba.fwd_block_finalize(qd, blocks, [], st, reset=True, n_kv_heads=Hkv, split_mode=split_mode)
        torch.cuda.synchronize()
        assert not H.host(out).any()
        assert np.all(np.isneginf(H.host(lse)))
