"""The C ABI under HIP graph capture: every entry point launches on the
caller's stream, allocates nothing and synchronises nothing, so a sequence of
calls can be captured once and replayed.  The test captures a ring step of
several fwd_block calls ending in fwd_block_finalize, and a fan-out decode,
replays the graph three times with other eager work on the stream in between,
and checks every replay bit for bit against the same calls run eagerly (the
kernels are deterministic).  Every case prints its name before it touches the
GPU."""

from __future__ import annotations

import pytest
import torch

from exact_blockwise_long_amd import blockattn as ba
from exact_blockwise_long_amd import synth
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


def test_ring_step_and_fanout_replayed_from_a_graph():
    seed = 91
    announce(f"graph capture: 4-visit ring step (split and walk) + fan-out decode, seed {seed}")
    g = synth.rng(seed)
    # A ring step on the walk (one call per visit, the last one finalising) ...
    T, Hq, Hkv, D, lens, q_pos0 = 4096, 16, 2, 128, [512, 700, 300, 536], 1500
    q = H.to_device(synth.normal(g, (T, Hq, D), 0.5, "bf16"))
    k = H.to_device(synth.normal(g, (sum(lens), Hkv, D), 0.5, "bf16"))
    v = H.to_device(synth.normal(g, (sum(lens), Hkv, D), 0.5, "bf16"))
    blocks, off = [], 0
    for n in lens:
        blocks.append((k[off:off + n], v[off:off + n], off))
        off += n
    order = [2, 1, 0, 3]
    # ... a short query block on the split path, with its workspace ...
    qs_ = H.to_device(synth.normal(g, (40, Hq, D), 0.5, "bf16"))
    kw_s = dict(n_kv_heads=Hkv, q_pos0=2000, causal=True)
    ws_s = torch.empty(max(16, ba.fwd_workspace_bytes(qs_, blocks, order, **kw_s)), dtype=torch.uint8,
                       device="cuda").fill_(0xFF)
    # ... and a fan-out decode.
    nb, P, S = 8, 3000, 100
    fq = H.to_device(synth.normal(g, (nb, Hq, D), 0.5, "bf16"))
    pk = H.to_device(synth.normal(g, (P, Hkv, D), 0.5, "bf16"))
    pv = H.to_device(synth.normal(g, (P, Hkv, D), 0.5, "bf16"))
    sk = H.to_device(synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16"))
    sv = H.to_device(synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16"))
    ws_f = torch.empty(ba.fanout_workspace_bytes(nb, Hq, Hkv, D, P, S), dtype=torch.uint8, device="cuda").fill_(0xFF)

    st = ba.new_state(T * Hq, D)
    st_s = ba.new_state(40 * Hq, D)
    out = torch.empty(T * Hq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(T * Hq, dtype=torch.float32, device="cuda")
    out_s = torch.empty(40 * Hq, D, dtype=torch.bfloat16, device="cuda")
    lse_s = torch.empty(40 * Hq, dtype=torch.float32, device="cuda")
    out_f = torch.empty(nb, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse_f = torch.empty(nb, Hq, dtype=torch.float32, device="cuda")
    kw = dict(n_kv_heads=Hkv, q_pos0=q_pos0, causal=True)

    def step():
        for i, j in enumerate(order[:-1]):
            ba.fwd_block(q, blocks, [j], st, reset=(i == 0), **kw)
        ba.fwd_block_finalize(q, blocks, order[-1:], st, reset=False, out=out, lse=lse, **kw)
        ba.fwd_block_finalize(qs_, blocks, order, st_s, reset=True, out=out_s, lse=lse_s, workspace=ws_s, **kw_s)
        ba.fanout_prefix_decode(fq, pk, pv, sk, sv, workspace=ws_f, out=out_f, lse=lse_f)

    results = (out, lse, out_s, lse_s, out_f, lse_f)
    step()
    torch.cuda.synchronize()
    eager = [r.clone() for r in results]

    # Capture on a side stream (default priority), after a warm-up there.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for r in results:
            r.zero_()   # eager work between replays; the replay must rewrite every output
        graph.replay()
        torch.cuda.synchronize()
        for got, ref, name in zip(results, eager, ("out", "lse", "split out", "split lse", "fanout out",
                                                   "fanout lse")):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager run"
        print(f"    replay {rep}: all six outputs equal the eager run bit for bit", flush=True)
