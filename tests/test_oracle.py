"""The CPU oracle against its pins (no GPU)."""
import math

import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention as att
from tiled_attention_memory_amd import workloads as wl


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    assert pin(att)


def test_rows_sum_to_one_and_mask_is_exact_zero():
    q, k = pins.rand((40, 8), 1), pins.rand((40, 8), 2)
    rows = np.arange(40)
    p, lse = att.softmax_rows(att.masked_scores(q, k, 0.9, True, rows))
    assert np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-12)
    assert np.all(p[np.triu_indices(40, 1)] == 0.0)
    # LSE identity and bounds, with the scores formed here by explicit loops
    for i in range(40):
        s = [0.9 * sum(q[i, d] * k[j, d] for d in range(8)) for j in range(i + 1)]
        assert abs(sum(math.exp(x - lse[i]) for x in s) - 1.0) < 1e-12
        assert max(s) <= lse[i] + 1e-12 and lse[i] <= max(s) + math.log(i + 1) + 1e-12


def test_delta_equals_rowwise_do_dot_o():
    B, hq, hkv, S, D = 1, 4, 2, 23, 8
    q, k, v, do = (pins.rand((B, hq, S, D), 3), pins.rand((B, hkv, S, D), 4),
                   pins.rand((B, hkv, S, D), 5), pins.rand((B, hq, S, D), 6))
    r = att.backward(q, k, v, do, 0.35, causal=True)
    assert pins.close(r["delta"], (r["o"] * do).sum(axis=-1), 1e-12)


def test_row_panels_equal_whole_matrix():
    B, hq, hkv, S, D = 1, 2, 1, 100, 8
    q, k, v, do = (pins.rand((B, hq, S, D), 7), pins.rand((B, hkv, S, D), 8),
                   pins.rand((B, hkv, S, D), 9), pins.rand((B, hq, S, D), 10))
    for causal in (True, False):
        whole = att.backward(q, k, v, do, 0.3, causal=causal)
        panel = att.backward(q, k, v, do, 0.3, causal=causal, panel_rows=16)
        for name in whole:
            assert pins.close(panel[name], whole[name], 1e-12), name


def test_group_subset_matches_full():
    B, hq, hkv, S, D = 2, 4, 2, 19, 8
    q, k, v, do = (pins.rand((B, hq, S, D), 11), pins.rand((B, hkv, S, D), 12),
                   pins.rand((B, hkv, S, D), 13), pins.rand((B, hq, S, D), 14))
    full = att.backward(q, k, v, do, 0.5)
    sub = att.backward(q, k, v, do, 0.5, heads=[(1, 0)])
    assert pins.close(sub["dk"][1, 0], full["dk"][1, 0], 1e-13)
    assert pins.close(sub["dq"][1, :2], full["dq"][1, :2], 1e-13)
    assert np.all(np.isnan(sub["dq"][0]))


def test_sampled_rows_and_columns_match_full():
    B, hq, hkv, S, D = 1, 4, 1, 64, 8
    q, k, v, do = (pins.rand((B, hq, S, D), 15), pins.rand((B, hkv, S, D), 16),
                   pins.rand((B, hkv, S, D), 17), pins.rand((B, hq, S, D), 18))
    scale = 0.4
    for causal in (True, False):
        full = att.backward(q, k, v, do, scale, causal=causal)
        rows = np.array([0, 5, 31, 63])
        for h in range(hq):
            r = att.rows_forward_backward(q[0, h], k[0, 0], v[0, 0], do[0, h], rows, scale, causal)
            for name in ("o", "lse", "delta", "dq"):
                assert pins.close(r[name], full[name][0, h, rows], 1e-12)
        row_lo = 40 if causal else 0
        rr = np.arange(row_lo, S)
        per = [att.rows_forward_backward(q[0, h], k[0, 0], v[0, 0], do[0, h], rr, scale, causal)
               for h in range(hq)]
        cols = np.array([40, 41, 50, 63])
        dk, dv = att.cols_dkdv(q[0, :, row_lo:], do[0, :, row_lo:], k[0, 0], v[0, 0], cols,
                               np.stack([p["lse"] for p in per]),
                               np.stack([p["delta"] for p in per]), row_lo, scale, causal)
        assert pins.close(dk, full["dk"][0, 0, cols], 1e-12)
        assert pins.close(dv, full["dv"][0, 0, cols], 1e-12)


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    vals = att.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -2.0
    assert vals[2] == 1.0 + 2.0 ** -7
    assert vals[3] == 2.0 ** -133
    assert vals[4] == (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert vals[5] == 0.0 and math.copysign(1.0, vals[5]) == -1.0


@pytest.mark.parametrize("w", [wl.WORKLOADS[0], wl.WORKLOADS[2]], ids=lambda w: w.name)
def test_oracle_matches_torch_on_workload_shapes(w):
    """The first and third workloads in full, from the seeded bf16 inputs, against torch fp64."""
    x = wl.workload_inputs(w)
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    r = att.backward(q, k, v, do, w.scale, causal=True)
    t = pins.torch_reference(q, k, v, do, w.scale, True)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert pins.close(r[name], t[name], 1e-9), name
