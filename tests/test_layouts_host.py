"""Host logic of the load-balanced causal shares against the oracle's
definitions of the layouts ([RAC] section 5) -- no GPU needed."""

from __future__ import annotations

import numpy as np
import pytest

from exact_blockwise_long_amd import layouts as L
from oracle import attention as ora

OWNERS = {"contiguous": ora.contiguous_tokens, "zigzag": ora.zigzag_tokens, "striped": ora.striped_tokens}


@pytest.mark.parametrize("layout", L.LAYOUTS)
@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_owned_tokens_match_the_oracle(layout, n):
    S = 8 * n
    for k in range(n):
        got = L.tokens(L.owned(layout, S, n, k))
        np.testing.assert_array_equal(got, OWNERS[layout](S, n, k))


@pytest.mark.parametrize("layout", L.LAYOUTS)
@pytest.mark.parametrize("n", [2, 3, 4])
def test_step_calls_compute_the_causal_pairs(layout, n):
    """Pairs the kernel would compute in its positions == causal pairs in absolute positions."""
    S = 12 * n
    for k in range(n):
        for t in range(n):
            assert L.step_pairs(layout, S, n, k, t) == ora.ring_step_pairs(OWNERS[layout], S, n, k, t), (k, t)


@pytest.mark.parametrize("n", [2, 3, 5])
def test_striped_positions_keep_the_causal_rule(n):
    B = 7
    S = n * B
    for k in range(n):
        for t in range(n):
            (c,) = L.step_calls("striped", S, n, k, t)
            (kv, pos0), = c.blocks
            for i in range(B):
                for j in range(B):
                    kernel_visible = pos0 + j <= c.q_pos0 + i
                    true_visible = kv.start + j * kv.step <= c.q.start + i * c.q.step
                    assert kernel_visible == true_visible, (k, t, i, j)


def test_ring_sources_follow_the_ring_order():
    for n in (1, 4, 7):
        for k in range(n):
            assert [L.source(n, k, t) for t in range(n)] == ora.ring_order(k, n)


def test_bad_layouts_are_rejected():
    with pytest.raises(ValueError):
        L.owned("diagonal", 16, 4, 0)
    with pytest.raises(ValueError):
        L.owned("zigzag", 12, 4, 0)   # 2N = 8 does not divide 12
    with pytest.raises(ValueError):
        L.owned("striped", 16, 4, 4)
