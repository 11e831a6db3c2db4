"""GPU parity of blockattn_merge_states over the part counts, head dims and
row counts that change the kernel's layout, against the oracle's log-sum-exp
merge in fp64 ("AHBM Agentic Runtime Architecture", s.3.4).

The kernel spreads the parts of a row over 1, 2, 4, 8 (D = 128) or up to 16
(D = 64) slices of a workgroup and combines the slices through LDS; with few
parts the slices cover more rows instead.  The cases reach every slice count,
the 64-part maximum and row counts that leave a ragged last workgroup.  The
states are synthetic: m ~ N(0, 8^2) with some -inf entries (parts that saw no
key), l in [0.5, 1.5), O ~ N(0, 1), all fp32; some rows are empty in every
part.  m is a max, so it must match exactly; l and O/l within fp32 rounding
of a sum of at most 64 terms.  Every case prints its name before it touches
the GPU.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_blockwise_long_amd import blockattn as ba
from oracle import attention as ora
from tests import helpers as H

pytestmark = pytest.mark.gpu

MAX_PARTS = 64   # BLOCKATTN_MAX_MERGE_PARTS


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ba.load()
    yield
    torch.cuda.synchronize()


def make_parts(seed, n_parts, rows, D):
    g = np.random.Generator(np.random.PCG64(seed))
    parts = []
    for _ in range(n_parts):
        m = (g.standard_normal(rows) * 8.0).astype(np.float32)
        m[g.random(rows) < 0.15] = -np.inf
        l = (g.random(rows) + 0.5).astype(np.float32)
        o = g.standard_normal((rows, D)).astype(np.float32)
        parts.append((m, l, o))
    # rows 0 and rows - 1 saw no key in any part
    for m, l, o in parts:
        m[[0, rows - 1]] = -np.inf
        l[[0, rows - 1]] = 0.0
        o[[0, rows - 1]] = 0.0
    return parts


# (n_parts, D, rows): slices per row 1, 1, 2, 4, 8, 8, 8 at D = 128 and 1, 4, 16 at D = 64.
CASES = [(1, 128, 37), (2, 128, 1001), (5, 128, 1003), (9, 128, 333), (17, 128, 515), (33, 128, 4097),
         (MAX_PARTS, 128, 2049), (2, 64, 1001), (9, 64, 777), (MAX_PARTS, 64, 999)]


@pytest.mark.parametrize("n_parts,D,rows", CASES, ids=[f"p{c[0]}_d{c[1]}_r{c[2]}" for c in CASES])
def test_merge_matches_oracle(n_parts, D, rows):
    seed = 7000 + 97 * n_parts + D + rows
    announce(f"merge_states n_parts={n_parts} D={D} rows={rows} seed {seed}")
    parts = make_parts(seed, n_parts, rows, D)
    m_ref, l_ref, o_ref = ora.merge([tuple(x.astype(np.float64) for x in p) for p in parts])
    dev = [tuple(torch.from_numpy(x).cuda() for x in p) for p in parts]
    out = ba.new_state(rows, D)
    ba.merge_states(dev, out)
    torch.cuda.synchronize()
    m, l, o = (H.host(x) for x in out)
    assert np.array_equal(m, m_ref.astype(np.float32)), "merged m must be the exact max"
    H.assert_close(l, l_ref, 2e-6 * n_parts, "merged l", rel=True)
    live = l_ref > 0
    with np.errstate(invalid="ignore", divide="ignore"):
        a = o[live] / l[live][:, None]
        a_ref = o_ref[live] / l_ref[live][:, None]
    H.assert_close(a, a_ref, 2e-6 * n_parts, "merged O / l")
    assert not o[~live].any() and not l[~live].any(), "rows with no key must stay l = 0, O = 0"

    # In place over the last part: the same values bit for bit.
    ba.merge_states(dev, dev[-1])
    torch.cuda.synchronize()
    for x, y, name in zip(dev[-1], out, "mlo"):
        assert torch.equal(x, y), f"in-place merge differs in {name}"
