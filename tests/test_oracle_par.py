"""The threaded oracle driver (oracle_par) against the oracle called directly.

oracle_par only distributes calls of the oracle's own functions over threads
and reassembles the results; here its outputs must equal the direct,
single-call oracle to rounding (the row-panel and column-block routes sum in
a different order), on a ragged causal shape with several panels and blocks
and on a non-causal one.
"""
import numpy as np
import pytest

import oracle_par as par
from oracle import attention as att


def _inputs(B, Hq, Hkv, S, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, S, D)), rng.standard_normal((B, Hkv, S, D)),
            rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hq, S, D)))


@pytest.mark.parametrize("causal", [True, False])
def test_groups_backward_equals_backward(causal):
    q, k, v, do = _inputs(2, 6, 2, 77, 16, 1)
    scale = 0.3
    want = att.backward(q, k, v, do, scale, causal=causal)
    groups = [(1, 1), (0, 0)]
    got = par.groups_backward(q, k, v, do, scale, causal, groups, panel_rows=20)
    for (b, kvh), r in zip(groups, got):
        hs = slice(3 * kvh, 3 * kvh + 3)
        for n in ("o", "lse", "delta", "dq"):
            np.testing.assert_allclose(r[n], want[n][b, hs], rtol=0, atol=1e-12)
        for n in ("dk", "dv"):
            np.testing.assert_allclose(r[n], want[n][b, kvh], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_rows_and_key_blocks_equal_backward(causal):
    q, k, v, do = _inputs(1, 3, 1, 203, 8, 2)
    scale = 0.25
    want = att.backward(q, k, v, do, scale, causal=causal)
    rows = par.all_rows(q[0], k[0, 0], v[0, 0], do[0], scale, panel_rows=64, causal=causal)
    for n in ("o", "lse", "delta", "dq"):
        np.testing.assert_allclose(rows[n], want[n][0], rtol=0, atol=1e-12)
    blocks = [0, 1, 6]   # the last block (192..202) is ragged
    kb = par.key_blocks_dkdv(q[0], do[0], k[0, 0], v[0, 0], rows["lse"], rows["delta"], blocks, 32,
                             scale, causal=causal)
    for j in blocks:
        sl = slice(32 * j, min(203, 32 * j + 32))
        np.testing.assert_allclose(kb[j][0], want["dk"][0, 0, sl], rtol=0, atol=1e-11)
        np.testing.assert_allclose(kb[j][1], want["dv"][0, 0, sl], rtol=0, atol=1e-11)
