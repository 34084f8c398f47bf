"""Seeded sweeps of the option paths against their oracles, every element.

Dropout (oracle.dropout, the same Philox bytes), rotary embedding (oracle.rope,
in both readings of the rotated inputs) and decoding against a cache
(oracle.blocks), each on shapes drawn from a fixed seed: sequence lengths at and
around the tiling edges, group sizes with and without head packing, both head
sizes and masks, probabilities, seeds and bases across their ranges.
"""
import math

import numpy as np
import pytest

from gpu_helpers import assert_close, assert_lse, say, to_f64
from oracle import attention as att
from oracle import blocks as blk
from oracle import dropout as dr
from oracle import rope
from test_decode import run_decode
from test_dropout import run as run_dropout
from test_rope import check_both_readings
from test_rope import run as run_rope
from tiled_attention_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu

EDGES = [1, 2, 31, 33, 63, 64, 65, 127, 129, 255, 257, 511, 512, 513, 600]


def _shape(rng, s_max=640):
    S = int(rng.choice(EDGES)) if rng.random() < 0.6 else int(rng.integers(1, s_max))
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 3, 4]))
    B = int(rng.choice([1, 2]))
    return B, Hkv * g, Hkv, S, D, bool(rng.random() < 0.75)


def _dropout_cases(n=12, seed=31):
    rng = np.random.default_rng(seed)
    return [(*_shape(rng), float(rng.choice([0.05, 0.2, 0.5, 0.75])), int(rng.integers(0, 1 << 63)))
            for _ in range(n)]


def _rope_cases(n=10, seed=32):
    rng = np.random.default_rng(seed)
    return [(*_shape(rng), float(rng.choice([1e4, 5e5, 1e6]))) for _ in range(n)]


def _decode_cases(n=10, seed=33):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8]))
        Sq = int(rng.choice([s for s in (1, 2, 4, 8, 16) if g * s <= 128]))
        Sk = int(rng.integers(Sq, 5000))
        out.append((int(rng.choice([1, 2])), Hkv * g, Hkv, Sq, Sk, D, bool(rng.random() < 0.8)))
    return out


@pytest.mark.parametrize("case", _dropout_cases(), ids=lambda c: "B{}_Hq{}_Hkv{}_S{}_D{}_{}_p{}".format(
    *c[:5], "causal" if c[5] else "full", c[6]))
def test_dropout_sweep(case):
    B, Hq, Hkv, S, D, causal, p, seed = case
    say(f"dropout sweep {case}")
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(931, B, Hq, S, D))
    scale = 1.0 / math.sqrt(D)
    g = run_dropout(x, causal, scale, p, seed)
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = dr.backward(q, k, v, do, scale, causal, p, seed)
    for name in ("o", "dq", "dk", "dv"):
        assert_close(name, to_f64(g[name]), ref[name])
    assert_lse(to_f64(g["lse"]), ref["lse"])


@pytest.mark.parametrize("case", _rope_cases(), ids=lambda c: "B{}_Hq{}_Hkv{}_S{}_D{}_{}_base{:g}".format(
    *c[:5], "causal" if c[5] else "full", c[6]))
def test_rope_sweep(case):
    B, Hq, Hkv, S, D, causal, base = case
    say(f"rope sweep {case}")
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(932, B, Hq, S, D))
    scale = 1.0 / math.sqrt(D)
    g = run_rope(x, causal, scale, base)
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    rnd = rope.backward(q, k, v, do, scale, causal, base, bf16_rotated=True)
    ext = rope.backward(q, k, v, do, scale, causal, base, bf16_rotated=False)
    # both readings, with their allowances (tests/test_rope.py)
    check_both_readings(g, q, k, rnd, ext, scale, causal, base, Hq // Hkv)


@pytest.mark.parametrize("case", _decode_cases(), ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Sk{}_D{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_decode_sweep(case):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    say(f"decode sweep {case}")
    x = wl.make_inputs(B, Hq, Hkv, Sk, D, seed=(933, B, Hq, Sq, Sk, D))
    scale = 1.0 / math.sqrt(D)
    go, gl = run_decode(x, Sq, causal, scale)
    q, k, v = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v"))
    ro, rl = blk.forward_block(q[:, :, Sk - Sq:], k, v, scale, causal, Sk - Sq, 0)
    assert_close("o", go, ro)
    assert_lse(gl, rl)
