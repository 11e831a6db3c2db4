"""GPU parity of the load-balanced causal shares ([RAC] section 5).

Every emulated device of a 4-device causal ring runs its ring steps through
the C ABI (one fwd_block call per query span and step, on views of the full
sequence) and must reproduce the oracle's plain causal attention for the
tokens that device holds, in absolute positions.  Chunks of 80 tokens span
one full 64-key tile and a ragged one; both key-split and walk modes run.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_blockwise_long_amd import blockattn as ba
from exact_blockwise_long_amd import layouts as L
from exact_blockwise_long_amd import synth
from oracle import attention as ora
from tests import helpers as H

pytestmark = pytest.mark.gpu

OWNERS = {"contiguous": ora.contiguous_tokens, "zigzag": ora.zigzag_tokens, "striped": ora.striped_tokens}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ba.load()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("split_mode", [1, 2])
@pytest.mark.parametrize("layout", L.LAYOUTS)
def test_layout_devices_match_causal_attention(layout, split_mode):
    n, Hq, Hkv, D = 4, 8, 2, 128
    S = 2 * n * 80
    print(f"[case] layout {layout} n={n} S={S} Hq={Hq} Hkv={Hkv} D={D} split_mode={split_mode} seed 73", flush=True)
    g = synth.rng(73)
    q = synth.normal(g, (S, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (S, Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (S, Hkv, D), 0.5, "bf16")
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    scale = 1.0 / np.sqrt(D)
    for dev in range(n):
        out, lse = L.run_device(ba, torch, layout, qd, kd, vd, n, dev, n_kv_heads=Hkv, split_mode=split_mode)
        torch.cuda.synchronize()
        mine = OWNERS[layout](S, n, dev)
        a_ref, _, _, lse_ref = ora.attend(q.f64()[mine], k.f64(), v.f64(), scale, mine, np.arange(S), True)
        H.assert_bf16_out(H.host(out), a_ref, f"{layout} device {dev}")
        H.assert_close(H.host(lse), lse_ref, H.BF16_LSE, f"{layout} device {dev} lse")
