"""Load-balanced causal shares as visit patterns on one GPU.

"RingAttention and Context Parallelism" (llms.blog), section 5 ("Causal
Masking and Load Balancing: Striped vs. Zigzag Ring Attention"): with causal
attention and contiguous shards, device k of N computes k + 1 of its N ring
steps and idles the rest.  Two layouts even the work out:

* zigzag -- the sequence is cut into 2N chunks; device k holds chunks k and
  2N - 1 - k, so every device has one early and one late chunk;
* striped -- device k holds every token whose index is k modulo N.

At ring step t device k holds the K/V of device (k - t) mod N (section 3).
This module turns (layout, N, device, step) into ``blockattn_fwd_block``
calls on views of the full sequence, so one GPU runs exactly the work one
device of the ring would run, shard by shard.  No tensor is copied: a chunk
is a slice and a stripe is a strided view.

Positions.  Contiguous and zigzag shards keep absolute positions.  For a
stripe, query i of device k sits at k + i*N and key j of device s at
s + j*N, so key j is visible to query i exactly when j + [s > k] <= i; the
calls therefore give the kernel query positions 0, 1, ... and key positions
[s > k], 1 + [s > k], ..., which keeps the kernel's causal rule (key
position <= query position) and its skipping of wholly-future tiles.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

LAYOUTS = ("contiguous", "zigzag", "striped")


@dataclass(frozen=True)
class Span:
    """Tokens start, start + step, ..., count of them."""
    start: int
    count: int
    step: int = 1

    def indices(self) -> List[int]:
        return [self.start + i * self.step for i in range(self.count)]


@dataclass(frozen=True)
class Call:
    """One ``blockattn_fwd_block`` call: query span ``q_index`` of the device
    (its own state) against K/V spans, with the positions the kernel compares."""
    q_index: int
    q: Span
    q_pos0: int
    blocks: Tuple[Tuple[Span, int], ...]   # (K/V tokens, position of their first key)


def _check(layout: str, seq_len: int, n: int):
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}; expected one of {LAYOUTS}")
    parts = 2 * n if layout == "zigzag" else n
    if n < 1 or seq_len % parts != 0:
        raise ValueError(f"{layout}: sequence length {seq_len} is not a multiple of {parts}")


def owned(layout: str, seq_len: int, n: int, k: int) -> List[Span]:
    """The query (and K/V) spans device k of n holds, in storage order."""
    _check(layout, seq_len, n)
    if not 0 <= k < n:
        raise ValueError(f"device {k} out of range for {n} devices")
    if layout == "contiguous":
        b = seq_len // n
        return [Span(k * b, b)]
    if layout == "zigzag":
        c = seq_len // (2 * n)
        return [Span(k * c, c), Span((2 * n - 1 - k) * c, c)]
    return [Span(k, seq_len // n, n)]


def source(n: int, k: int, t: int) -> int:
    """The device whose K/V device k holds at ring step t."""
    return (k - t) % n


def step_calls(layout: str, seq_len: int, n: int, k: int, t: int) -> List[Call]:
    """The fwd_block calls of device k at ring step t, one per query span."""
    src = source(n, k, t)
    mine = owned(layout, seq_len, n, k)
    theirs = owned(layout, seq_len, n, src)
    if layout == "striped":
        off = 1 if src > k else 0
        return [Call(0, mine[0], 0, ((theirs[0], off),))]
    kv = tuple((sp, sp.start) for sp in theirs)
    return [Call(i, sp, sp.start, kv) for i, sp in enumerate(mine)]


def _view(x, sp: Span):
    return x[sp.start: sp.start + (sp.count - 1) * sp.step + 1: sp.step]


def run_device(ba, torch, layout: str, q, k, v, n: int, dev: int, *, n_kv_heads: int, scale: float = 0.0,
               split_mode: int = 0, calls_out: list | None = None):
    """Emulates device ``dev`` of an n-device causal ring on the full-sequence
    tensors q [S, Hq, D], k and v [S, Hkv, D]: its n steps of fwd_block calls,
    then finalize.  Returns (out [tokens held, Hq, D] bf16, lse [tokens held, Hq])
    in the device's storage order.  ``calls_out`` collects one zero-argument
    callable per (step, call) for timing."""
    S, Hq, D = q.shape
    spans = owned(layout, S, n, dev)
    states = [ba.new_state(sp.count * Hq, D) for sp in spans]
    for t in range(n):
        for c in step_calls(layout, S, n, dev, t):
            qv = _view(q, c.q)
            blocks = [(_view(k, sp), _view(v, sp), pos0) for sp, pos0 in c.blocks]

            def call(qv=qv, blocks=blocks, st=states[c.q_index], reset=(t == 0), p0=c.q_pos0):
                ba.fwd_block(qv, blocks, None, st, reset, n_kv_heads=n_kv_heads, q_pos0=p0, causal=True,
                             scale=scale, split_mode=split_mode)

            call()
            if calls_out is not None:
                calls_out.append((t, call))
    outs, lses = [], []
    for sp, st in zip(spans, states):
        o, lse = ba.finalize(st)
        outs.append(o.view(sp.count, Hq, D))
        lses.append(lse.view(sp.count, Hq))
    return torch.cat(outs, 0), torch.cat(lses, 0)


def visible_pairs_of_call(c: Call) -> int:
    """Causal (query, key) pairs one call computes, in the kernel's positions."""
    total = 0
    for sp, pos0 in c.blocks:
        for i in range(c.q.count):
            qp = c.q_pos0 + i
            total += max(0, min(sp.count, qp - pos0 + 1))
    return total


def step_pairs(layout: str, seq_len: int, n: int, k: int, t: int) -> int:
    return sum(visible_pairs_of_call(c) for c in step_calls(layout, seq_len, n, k, t))


def tokens(spans: Sequence[Span]) -> List[int]:
    return [i for sp in spans for i in sp.indices()]
