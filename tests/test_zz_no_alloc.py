"""The allocation-free fan-out decode (fanout_prefix_decode_noalloc, through
the C ABI) against fanout_prefix_decode with a caller workspace: the same
kernels, so the outputs must be equal bit for bit.  Two calls in a row on the
same static scratch, the second with a smaller input, each checked; the
full-size one is also checked against the oracle on sampled rows.
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


def inputs(seed, nb, Hq, Hkv, D, P, S):
    g = synth.rng(seed)
    q = synth.normal(g, (nb, Hq, D), 0.5, "bf16")
    pk = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    pv = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    sk = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    sv = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    return q, pk, pv, sk, sv


def nan_like(t):
    return torch.empty_like(t).view(torch.uint8).fill_(0xFF).view(t.dtype)


def test_noalloc_decode_matches_workspace_decode_twice():
    w = wl.FANOUT_DECODE
    cases = [
        ("full-size 64K decode", w.seed, w.n_branches, w.n_q_heads, w.n_kv_heads, w.head_dim, w.prefix_len,
         w.suffix_len),
        ("smaller decode", 91, 3, 16, 2, 128, 1000, 100),
    ]
    for name, seed, nb, Hq, Hkv, D, P, S in cases:
        announce(f"noalloc {name}: nb {nb} Hq {Hq} Hkv {Hkv} D {D} P {P} S {S} seed {seed}")
        host = inputs(seed, nb, Hq, Hkv, D, P, S)
        dev = [H.to_device(t) for t in host]
        ref_out, ref_lse = ba.fanout_prefix_decode(*dev)
        out = nan_like(ref_out)
        lse = nan_like(ref_lse)
        ba.fanout_prefix_decode_noalloc(*dev, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"{name}: output differs from fanout_prefix_decode"
        assert torch.equal(lse, ref_lse), f"{name}: lse differs from fanout_prefix_decode"
        # and the oracle, on a sample of branches (all of them for the small case)
        branches = list(range(nb)) if nb <= 4 else [0, nb // 2, nb - 1]
        q, pk, pv, sk, sv = host
        a_ref, lse_ref = ora.fanout_decode(q.f64()[branches], pk.f64(), pv.f64(), sk.f64()[branches],
                                           sv.f64()[branches], 1.0 / np.sqrt(D))
        H.assert_bf16_out(H.host(out)[branches], a_ref, name)
        H.assert_close(H.host(lse)[branches], lse_ref, H.BF16_LSE, name + " lse")


def test_noalloc_rejects_more_than_the_scratch():
    nb, Hq, Hkv, D, P, S = 2048, 64, 8, 128, 65536, 512
    announce(f"noalloc beyond its scratch: nb {nb} P {P} S {S} (rejected on the host)")
    assert ba.fanout_workspace_bytes(nb, Hq, Hkv, D, P, S) > ba.STATIC_SCRATCH_BYTES
    q = torch.zeros(nb, Hq, D, dtype=torch.bfloat16, device="cuda")
    pk = torch.zeros(P, Hkv, D, dtype=torch.bfloat16, device="cuda")
    sk = torch.zeros(nb, S, Hkv, D, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(nb, Hq, D, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ba.BlockAttnError, match="static scratch"):
        ba.fanout_prefix_decode_noalloc(q, pk, pk, sk, sk, out=out)
