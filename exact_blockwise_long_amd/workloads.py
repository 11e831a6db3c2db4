"""The synthetic workloads of the blockwise-attention hot path, with their accounting.

Each workload is named for what it is.  Inputs are drawn by ``synth`` (seeded
PCG64 normals rounded once to bf16, or kept fp32).  Algorithmic work is the
minimum the method must do:

* FLOPs = 4 * D * (number of visible (query row, key) pairs), the two matrix
  products QK^T and PV of the per-step count 4 B^2 d in "RingAttention and
  Context Parallelism", section 4; masked pairs are not counted.
* Bytes = Q read once + every K/V row a query can see read once + the output
  (or, for state-producing steps, the state) written once.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np

from . import synth


@dataclass
class BlockwiseWorkload:
    """A stationary query block walking K/V blocks in a given order."""

    name: str
    dtype: str                  # "bf16" or "f32" (Q, K, V storage)
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    q_len: int
    q_pos0: int                 # absolute position of query row 0
    block_len: int
    n_blocks: int               # K/V blocks cover positions [0, n_blocks*block_len)
    order: List[int]
    causal: bool
    seed: int
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    note: str = ""

    @property
    def kv_len(self) -> int:
        return self.block_len * self.n_blocks

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def rows(self) -> int:
        return self.q_len * self.n_q_heads

    def visible_keys_per_row(self, block: int) -> np.ndarray:
        """Visible keys of ``block`` for each query token (length q_len)."""
        pos0 = block * self.block_len
        if not self.causal:
            return np.full(self.q_len, self.block_len, dtype=np.int64)
        q_pos = self.q_pos0 + np.arange(self.q_len, dtype=np.int64)
        return np.clip(q_pos - pos0 + 1, 0, self.block_len)

    def pairs(self) -> int:
        """Visible (query token, key) pairs over the visited blocks, per query head."""
        return int(sum(self.visible_keys_per_row(b).sum() for b in self.order))

    def flops(self) -> float:
        return 4.0 * self.head_dim * self.n_q_heads * self.pairs()

    def visited_nonempty(self) -> List[int]:
        return [b for b in self.order if self.visible_keys_per_row(b).max() > 0]

    def bytes(self) -> int:
        esz = 2 if self.dtype == "bf16" else 4
        q = self.q_len * self.n_q_heads * self.head_dim * esz
        kv = 2 * len(self.visited_nonempty()) * self.block_len * self.n_kv_heads * self.head_dim * esz
        out = self.q_len * self.n_q_heads * self.head_dim * esz
        return q + kv + out

    def make_inputs(self):
        """(q, k, v) synth.Tensors: q [q_len, Hq, D]; k, v [kv_len, Hkv, D]."""
        g = synth.rng(self.seed)
        q = synth.normal(g, (self.q_len, self.n_q_heads, self.head_dim), self.q_scale, self.dtype)
        k = synth.normal(g, (self.kv_len, self.n_kv_heads, self.head_dim), self.k_scale, self.dtype)
        v = synth.normal(g, (self.kv_len, self.n_kv_heads, self.head_dim), self.v_scale, self.dtype)
        return q, k, v

    def make_dout(self):
        """The gradient of a loss with respect to the output, [q_len, Hq, D], for
        backward workloads: N(0, 1) * q_scale from its own stream (seed + 1000)."""
        g = synth.rng(self.seed + 1000)
        return synth.normal(g, (self.q_len, self.n_q_heads, self.head_dim), self.q_scale, self.dtype)


@dataclass
class FanoutWorkload:
    """Shared-prefix fan-out decode: one new query token per branch."""

    name: str
    n_branches: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    prefix_len: int
    suffix_len: int
    seed: int
    q_scale: float = 0.5
    k_scale: float = 0.5
    v_scale: float = 0.5
    dtype: str = "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def rows(self) -> int:
        return self.n_branches * self.n_q_heads

    def flops(self) -> float:
        keys = self.prefix_len + self.suffix_len
        return 4.0 * self.head_dim * self.rows * keys

    def bytes(self) -> int:
        e = 2
        q = self.rows * self.head_dim * e
        prefix = 2 * self.prefix_len * self.n_kv_heads * self.head_dim * e
        suffix = 2 * self.n_branches * self.suffix_len * self.n_kv_heads * self.head_dim * e
        out = self.rows * self.head_dim * e
        return q + prefix + suffix + out

    def make_inputs(self):
        """q [nb, Hq, D], prefix k/v [P, Hkv, D], suffix k/v [nb, S, Hkv, D], drawn in that order."""
        g = synth.rng(self.seed)
        D, Hq, Hkv = self.head_dim, self.n_q_heads, self.n_kv_heads
        q = synth.normal(g, (self.n_branches, Hq, D), self.q_scale, self.dtype)
        pk = synth.normal(g, (self.prefix_len, Hkv, D), self.k_scale, self.dtype)
        pv = synth.normal(g, (self.prefix_len, Hkv, D), self.v_scale, self.dtype)
        sk = synth.normal(g, (self.n_branches, self.suffix_len, Hkv, D), self.k_scale, self.dtype)
        sv = synth.normal(g, (self.n_branches, self.suffix_len, Hkv, D), self.v_scale, self.dtype)
        return q, pk, pv, sk, sv


@dataclass
class ShardMergeWorkload:
    """Per-shard partial states of a few query rows, then an n-way LSE merge.

    The query rows are ``n_branches`` tokens x ``n_q_heads`` heads of one KV
    head group; the K/V sequence of that group is split into ``n_shards``
    contiguous shards.
    """

    name: str
    n_branches: int
    n_q_heads: int
    head_dim: int
    kv_len: int
    n_shards: int
    seed: int
    q_scale: float = 0.5
    k_scale: float = 12.0
    v_scale: float = 0.5
    dtype: str = "bf16"
    n_kv_heads: int = 1

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def shard_len(self) -> int:
        return self.kv_len // self.n_shards

    @property
    def rows(self) -> int:
        return self.n_branches * self.n_q_heads

    def flops(self) -> float:
        return 4.0 * self.head_dim * self.rows * self.kv_len

    def sweep_bytes(self) -> int:
        """K/V read once + Q read + every shard's fp32 partial written once and read once."""
        kv = 2 * self.kv_len * self.n_kv_heads * self.head_dim * 2
        q = self.rows * self.head_dim * 2
        partials = 2 * self.n_shards * self.rows * (self.head_dim + 2) * 4
        out = self.rows * self.head_dim * 2
        return kv + q + partials + out

    def merge_bytes(self) -> int:
        return (self.n_shards + 1) * self.rows * (self.head_dim + 2) * 4

    def make_inputs(self):
        """q [nb, Hq, D]; k, v [kv_len, 1, D]; drawn Q, K, V."""
        g = synth.rng(self.seed)
        q = synth.normal(g, (self.n_branches, self.n_q_heads, self.head_dim), self.q_scale, self.dtype)
        k = synth.normal(g, (self.kv_len, self.n_kv_heads, self.head_dim), self.k_scale, self.dtype)
        v = synth.normal(g, (self.kv_len, self.n_kv_heads, self.head_dim), self.v_scale, self.dtype)
        return q, k, v


def ring_order(k: int, n: int) -> List[int]:
    """Blocks device k visits, (k - t) mod n at step t (ring direction of the llms.blog page, section 3)."""
    return [(k - t) % n for t in range(n)]


TINY_EXACT = BlockwiseWorkload(
    name="tiny_exact_f32: 1 head, D64, fp32, 256 queries vs 4 blocks of 256 keys, order 1,2,3,0",
    dtype="f32", n_q_heads=1, n_kv_heads=1, head_dim=64, q_len=256, q_pos0=0,
    block_len=256, n_blocks=4, order=[1, 2, 3, 0], causal=False, seed=1)

CAUSAL_PREFILL = BlockwiseWorkload(
    name="causal_prefill_32k: bf16 GQA 64/8 D128, query block 7 of 8x4096, causal",
    dtype="bf16", n_q_heads=64, n_kv_heads=8, head_dim=128, q_len=4096, q_pos0=7 * 4096,
    block_len=4096, n_blocks=8, order=ring_order(7, 8), causal=True, seed=2,
    q_scale=0.5, k_scale=0.5, v_scale=0.5)

RING_SHARE = BlockwiseWorkload(
    name="ring_share_256k: bf16 GQA 64/8 D128, query block 12 of 16x16384, causal, one call per visit",
    dtype="bf16", n_q_heads=64, n_kv_heads=8, head_dim=128, q_len=16384, q_pos0=12 * 16384,
    block_len=16384, n_blocks=16, order=ring_order(12, 16), causal=True, seed=3,
    q_scale=0.5, k_scale=0.5, v_scale=0.5)

FANOUT_DECODE = FanoutWorkload(
    name="fanout_decode_64k: bf16 GQA 64/8 D128, prefix 65536, 16 branches x 512 suffix, 1 token each",
    n_branches=16, n_q_heads=64, n_kv_heads=8, head_dim=128, prefix_len=65536,
    suffix_len=512, seed=4)

SHARD_MERGE = ShardMergeWorkload(
    name="shard_merge_1m: bf16 D128, 8 branches x 8 heads of one KV group, 1048576 keys in 32 shards, logits ~ +-30",
    n_branches=8, n_q_heads=8, head_dim=128, kv_len=1048576, n_shards=32, seed=5)

@dataclass
class FanoutPrefillWorkload:
    """Shared-prefix fan-out over the newest T tokens of every branch (prefill
    of the private suffixes): each new token sees the prefix and its branch's
    suffix up to itself."""

    name: str
    n_branches: int
    n_new: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    prefix_len: int
    suffix_len: int
    seed: int
    scale_qkv: float = 0.5

    def pairs(self) -> int:
        """Visible (query token, key) pairs, per query head."""
        T, P, S = self.n_new, self.prefix_len, self.suffix_len
        per_branch = sum(P + S - T + i + 1 for i in range(T))
        return self.n_branches * per_branch

    def flops(self) -> float:
        return 4.0 * self.head_dim * self.n_q_heads * self.pairs()

    def bytes(self) -> int:
        kv_tok = 2 * self.n_kv_heads * self.head_dim * 2
        q = self.n_branches * self.n_new * self.n_q_heads * self.head_dim * 2
        return self.prefix_len * kv_tok + self.n_branches * self.suffix_len * kv_tok + 2 * q

    def make_inputs(self):
        """(q [nb, T, Hq, D], prefix_k, prefix_v [P, Hkv, D], suffix_k, suffix_v [nb, S, Hkv, D])."""
        g = synth.rng(self.seed)
        nb, T, Hq, Hkv, D = self.n_branches, self.n_new, self.n_q_heads, self.n_kv_heads, self.head_dim
        q = synth.normal(g, (nb, T, Hq, D), self.scale_qkv, "bf16")
        pk = synth.normal(g, (self.prefix_len, Hkv, D), self.scale_qkv, "bf16")
        pv = synth.normal(g, (self.prefix_len, Hkv, D), self.scale_qkv, "bf16")
        sk = synth.normal(g, (nb, self.suffix_len, Hkv, D), self.scale_qkv, "bf16")
        sv = synth.normal(g, (nb, self.suffix_len, Hkv, D), self.scale_qkv, "bf16")
        return q, pk, pv, sk, sv


@dataclass
class CausalRingWorkload:
    """A whole causal sequence sharded over n emulated ring devices in one of
    the layouts of "RingAttention and Context Parallelism", section 5; every
    device's ring steps run on the one GPU."""

    name: str
    seq_len: int
    n_devices: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seed: int
    scale_qkv: float = 0.5

    def pairs(self) -> int:
        """Causal (query token, key) pairs of the whole sequence, per query head."""
        return self.seq_len * (self.seq_len + 1) // 2

    def flops(self) -> float:
        return 4.0 * self.head_dim * self.n_q_heads * self.pairs()

    def make_inputs(self):
        """(q, k, v) synth.Tensors over the whole sequence: q [S, Hq, D]; k, v [S, Hkv, D]."""
        g = synth.rng(self.seed)
        q = synth.normal(g, (self.seq_len, self.n_q_heads, self.head_dim), self.scale_qkv, "bf16")
        k = synth.normal(g, (self.seq_len, self.n_kv_heads, self.head_dim), self.scale_qkv, "bf16")
        v = synth.normal(g, (self.seq_len, self.n_kv_heads, self.head_dim), self.scale_qkv, "bf16")
        return q, k, v


FANOUT_PREFILL = FanoutPrefillWorkload(
    name="fanout_prefill_64k: bf16 GQA 64/8 D128, prefix 65536, 8 branches x 20 new tokens, 512-token private suffixes",
    n_branches=8, n_new=20, n_q_heads=64, n_kv_heads=8, head_dim=128, prefix_len=65536, suffix_len=512, seed=7)

CAUSAL_RING_LAYOUTS = CausalRingWorkload(
    name="causal_ring_32k_8dev: bf16 GQA 64/8 D128, 32768 tokens over 8 emulated devices "
         "(contiguous / zigzag / striped shards)",
    seq_len=32768, n_devices=8, n_q_heads=64, n_kv_heads=8, head_dim=128, seed=6)

ALL = [TINY_EXACT, CAUSAL_PREFILL, RING_SHARE, FANOUT_DECODE, SHARD_MERGE]


def paged_layout(g: np.random.Generator, n_branches: int, prefix_len: int, suffix_len: int, page_len: int,
                 extra_pages: int = 3):
    """Seeded page tables for a paged fan-out: the prefix's ceil(P / page_len)
    pages and every branch's ceil(S / page_len) private pages at distinct pool
    pages in random order, plus ``extra_pages`` pages nothing refers to.
    Returns (n_pool, prefix_pages int32 [n_p], suffix_pages int32 [nb, n_s])."""
    n_p = -(-prefix_len // page_len)
    n_s = -(-suffix_len // page_len)
    n_pool = n_p + n_branches * n_s + extra_pages
    perm = g.permutation(n_pool).astype(np.int32)
    prefix_pages = perm[:n_p].copy()
    suffix_pages = perm[n_p:n_p + n_branches * n_s].reshape(n_branches, n_s).copy()
    return n_pool, prefix_pages, suffix_pages


# bf16 bit patterns that poison every key row no correct read touches: NaN,
# +inf, -inf and a negative NaN, cycled element by element.  A kernel that
# lets such a row into a result (even multiplied by a zero weight) shows NaN.
POISON_BF16 = np.array([0x7FC0, 0x7F80, 0xFF80, 0xFFC1], dtype=np.uint16)


def poison_rows(shape) -> np.ndarray:
    """A bf16 bit array of ``shape`` filled with the POISON_BF16 cycle."""
    n = int(np.prod(shape))
    return np.resize(POISON_BF16, n).reshape(shape)


def scatter_pages(g: np.random.Generator, prefix: synth.Tensor, suffix: synth.Tensor, n_pool: int,
                  prefix_pages: np.ndarray, suffix_pages: np.ndarray, page_len: int):
    """A bf16 page pool [n_pool, page_len, Hkv, D] holding ``prefix`` [P, Hkv, D]
    and each branch's ``suffix`` [nb, S, Hkv, D] at the given pages; every
    other row (unused pages, the tails of partial pages) holds NaN and +-inf
    (POISON_BF16), which no correct read touches.  ``g`` is not used."""
    tail = prefix.shape[1:] if prefix.shape[0] else suffix.shape[2:]
    pool = poison_rows((n_pool, page_len) + tuple(tail))

    def put(x, pages):
        for i, pid in enumerate(pages):
            rows = x[i * page_len:(i + 1) * page_len]
            pool[pid, :rows.shape[0]] = rows

    put(prefix.storage, prefix_pages)
    for b in range(suffix.shape[0]):
        put(suffix.storage[b], suffix_pages[b])
    return synth.Tensor(pool, "bf16")
