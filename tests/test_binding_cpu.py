"""The Python binding rejects tensors whose sizes do not match what the C ABI
will read or write (the library sees only pointers, so it cannot).  Every
case here raises before any library call is made; none reaches a kernel."""

from __future__ import annotations

import os

import pytest
import torch

from exact_blockwise_long_amd import blockattn as ba


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(ba.LIB_PATH):
        pytest.skip("libblockattn.so not built")
    ba.load()


def bf16(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def state(rows, D):
    return f32(rows), f32(rows), f32(rows, D)


def test_fwd_block_checks_blocks_and_state():
    q = bf16(16, 8, 128)
    good = (bf16(64, 2, 128), bf16(64, 2, 128), 0)
    with pytest.raises(ValueError, match="block 0"):
        ba.fwd_block(q, [(bf16(64, 1, 128), bf16(64, 1, 128), 0)], None, state(128, 128), True, n_kv_heads=2)
    with pytest.raises(ValueError, match="block 0"):
        ba.fwd_block(q, [(bf16(64, 2, 64), bf16(64, 2, 64), 0)], None, state(128, 128), True, n_kv_heads=2)
    with pytest.raises(ValueError, match="block 0"):
        ba.fwd_block(q, [(f32(64, 2, 128), f32(64, 2, 128), 0)], None, state(128, 128), True, n_kv_heads=2)
    with pytest.raises(ValueError, match="state"):
        ba.fwd_block(q, [good], None, state(64, 128), True, n_kv_heads=2)
    m, l, o = state(128, 128)
    with pytest.raises(ValueError, match="state.o"):
        ba.fwd_block(q, [good], None, (m, l, f32(128, 64)), True, n_kv_heads=2)
    m, l, o = state(128, 128)
    with pytest.raises(ValueError, match="state.o"):
        ba.fwd_block(q, [good], None, (m, l, o.to(torch.bfloat16)), True, n_kv_heads=2)


def test_shard_merge_finalize_check_states():
    q = bf16(4, 8, 128)
    blocks = [(bf16(64, 8, 128), bf16(64, 8, 128), 0)] * 2
    with pytest.raises(ValueError, match="one output state per block"):
        ba.shard_states(q, blocks, [state(32, 128)], n_kv_heads=8)
    with pytest.raises(ValueError, match=r"states_out\[1\]"):
        ba.shard_states(q, blocks, [state(32, 128), state(16, 128)], n_kv_heads=8)
    with pytest.raises(ValueError, match=r"parts\[0\]"):
        ba.merge_states([state(10, 128)], state(12, 128))
    with pytest.raises(ValueError, match="out must be"):
        ba.finalize(state(12, 128), out=bf16(11, 128))
    with pytest.raises(ValueError, match="lse must be"):
        ba.finalize(state(12, 128), lse=f32(13))


def test_backward_bindings_check_sizes():
    with pytest.raises(ValueError, match="row for row"):
        ba.bwd_delta(bf16(100, 128), bf16(99, 128))
    with pytest.raises(ValueError, match="delta must be"):
        ba.bwd_delta(bf16(100, 128), bf16(100, 128), delta=f32(50))
    q = bf16(16, 8, 128)
    blocks = [(bf16(64, 2, 128), bf16(64, 2, 128), 0)]
    dkv = [(f32(64, 2, 128), f32(64, 2, 128))]
    lse, delta, dq = f32(128), f32(128), f32(128, 128)
    with pytest.raises(ValueError, match="lse must be"):
        ba.bwd_block(q, bf16(16, 8, 128), lse.to(torch.bfloat16), delta, blocks, None, dq, dkv, n_kv_heads=2)
    with pytest.raises(ValueError, match="delta must be"):
        ba.bwd_block(q, bf16(16, 8, 128), lse, f32(64), blocks, None, dq, dkv, n_kv_heads=2)
    with pytest.raises(ValueError, match="dout must be"):
        ba.bwd_block(q, bf16(15, 8, 128), lse, delta, blocks, None, dq, dkv, n_kv_heads=2)
    with pytest.raises(ValueError, match="one .dk, dv. pair per block"):
        ba.bwd_block(q, bf16(16, 8, 128), lse, delta, blocks, None, dq, dkv * 2, n_kv_heads=2)
    with pytest.raises(ValueError, match="must have shape"):
        ba.bwd_block(q, bf16(16, 8, 128), lse, delta, blocks, None, dq, [(f32(63, 2, 128), f32(64, 2, 128))],
                     n_kv_heads=2)
    with pytest.raises(ValueError, match="block 0"):
        ba.bwd_block(q, bf16(16, 8, 128), lse, delta, [(bf16(64, 4, 128), bf16(64, 4, 128), 0)], None, dq, dkv,
                     n_kv_heads=2)


def test_fanout_bindings_check_shapes():
    q, pk, pv = bf16(4, 16, 128), bf16(100, 2, 128), bf16(100, 2, 128)
    sk, sv = bf16(4, 10, 2, 128), bf16(4, 10, 2, 128)
    with pytest.raises(ValueError, match="suffix_v"):
        ba.fanout_prefix_decode(q, pk, pv, sk, bf16(3, 10, 2, 128))
    with pytest.raises(ValueError, match="prefix_v"):
        ba.fanout_prefix_decode(q, pk, bf16(99, 2, 128), sk, sv)
    with pytest.raises(ValueError, match="out must be"):
        ba.fanout_prefix_decode(q, pk, pv, sk, sv, out=bf16(4, 16, 64))
    with pytest.raises(ValueError, match="lse must be"):
        ba.fanout_prefix_decode(q, pk, pv, sk, sv, lse=f32(4, 15))
    with pytest.raises(ValueError, match="in pairs"):
        ba.fanout_prefix_decode(q, pk, None, sk, sv)
    qp = bf16(4, 3, 16, 128)
    with pytest.raises(ValueError, match="out must be"):
        ba.fanout_prefix_prefill(qp, pk, pv, sk, sv, out=bf16(4, 16, 128))
    with pytest.raises(ValueError, match="suffix_k"):
        ba.fanout_prefix_prefill(qp, pk, pv, bf16(4, 10, 1, 128), sv)


def test_paged_fanout_bindings_check_pools_and_tables():
    q = bf16(4, 16, 128)
    pool = bf16(20, 64, 2, 128)
    pp = torch.zeros(16, dtype=torch.int32)          # 1000 prefix tokens / 64 = 16 pages
    sp = torch.zeros(4, 2, dtype=torch.int32)        # 100 suffix tokens / 64 = 2 pages per branch
    with pytest.raises(ValueError, match="same shape"):
        ba.fanout_prefix_decode_paged(q, pool, bf16(20, 64, 2, 64), pp, sp, 1000, 100)
    with pytest.raises(ValueError, match="prefix_pages"):
        ba.fanout_prefix_decode_paged(q, pool, pool, pp[:15], sp, 1000, 100)
    with pytest.raises(ValueError, match="prefix_pages"):
        ba.fanout_prefix_decode_paged(q, pool, pool, pp.to(torch.int64), sp, 1000, 100)
    with pytest.raises(ValueError, match="suffix_pages"):
        ba.fanout_prefix_decode_paged(q, pool, pool, pp, sp[:, :1], 1000, 100)
    with pytest.raises(ValueError, match="suffix_pages"):
        ba.fanout_prefix_decode_paged(q, pool, pool, pp, None, 1000, 100)
    with pytest.raises(ValueError, match="head_dim"):
        ba.fanout_prefix_decode_paged(bf16(4, 16, 64), pool, pool, pp, sp, 1000, 100)
    with pytest.raises(ValueError, match="out must be"):
        ba.fanout_prefix_decode_paged(q, pool, pool, pp, sp, 1000, 100, out=bf16(4, 16, 64))
    with pytest.raises(ValueError, match="lse must be"):
        ba.fanout_prefix_prefill_paged(bf16(4, 3, 16, 128), pool, pool, pp, sp, 1000, 100, lse=f32(4, 16))
