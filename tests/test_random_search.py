"""Seeded random search of every path against the oracles.

By default a fixed set: the first 40 cases of seed 4242, a few seconds. A longer search runs for
a given time instead:

    TAM_RANDOM_SEARCH_SECONDS=600 [TAM_RANDOM_SEARCH_SEED=4242] \
        python -u -m pytest tests/test_random_search.py -m gpu -s

Draws cases until the time is up, with shapes weighted to the tiling edges:
- the plain forward and backward, with scales, K x 3 and both masks;
- dropout, rotary embedding and decoding against a cache;
- the context-parallel block protocol with random cuts.

Each case is held to the same bounds as the fixed tests: the absolute bound on O and LSE, both
readings of RoPE with their allowances (tests/test_rope.py), and for dQ, dK and dV the normwise
bound of the fp16 gradient products, 2e-2 + 2^-10 max|x| (tests/test_special.py). Every case
prints one line. A failure prints its parameters, which rerun identically from the same seed.
"""
import math
import os
import time

import numpy as np
import pytest

from gpu_helpers import assert_close as _assert_close
from gpu_helpers import assert_lse, run_gpu, to_f64
from oracle import attention as att
from oracle import blocks as blk
from oracle import dropout as dr
from oracle import rope
from test_blocks import _cuts, run_blocks
from test_decode import run_decode
from test_dropout import run as run_dropout
from test_rope import check_both_readings
from test_rope import run as run_rope
from tiled_attention_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu

SECONDS = float(os.environ.get("TAM_RANDOM_SEARCH_SECONDS", "0"))
DEFAULT_CASES = 40
SEED = int(os.environ.get("TAM_RANDOM_SEARCH_SEED", "4242"))
EDGES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513, 640, 1023, 1024, 1025]


def assert_close(name, got, want):
    bound = 2e-2
    if name.startswith(("dq", "dk", "dv")):
        bound += 2.0 ** -10 * float(np.abs(np.asarray(want)).max())
    _assert_close(name, got, want, max_abs=bound)


class Search:
    def __init__(self, seed):
        self.seed = seed
        self.rng = np.random.default_rng(seed)

    def shape(self, smax=1100):
        r = self.rng
        S = int(r.choice(EDGES)) if r.random() < 0.5 else int(r.integers(1, smax))
        D = int(r.choice([64, 128]))
        Hkv = int(r.choice([1, 2, 3, 4]))
        g = int(r.choice([1, 2, 3, 4, 6, 8, 16]))
        B = int(r.choice([1, 2, 3]))
        # keep the oracle's work near 24 heads of 1100^2 scores
        while B * Hkv * g * S * S > 24 * 1100 * 1100 and (B > 1 or g > 1 or Hkv > 1):
            if B > 1:
                B -= 1
            elif g > 1:
                g = max(1, g // 2)
            else:
                Hkv -= 1
        return B, Hkv * g, Hkv, S, D, bool(r.random() < 0.7)

    def plain(self):
        B, Hq, Hkv, S, D, causal = self.shape()
        r = self.rng
        scale = 1.0 / math.sqrt(D) if r.random() < 0.7 else float(r.choice([0.05, 0.3, -0.2, 0.5]))
        km = float(r.choice([1.0, 1.0, 3.0]))
        desc = f"plain B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal={causal} scale={scale:.3g} k_mult={km}"
        x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(self.seed, 1, B, Hq, S, D), k_mult=km)

        def check():
            g = run_gpu(x, causal, scale)
            q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
            ref = att.backward(q, k, v, do, scale, causal=causal)
            for n in ("o", "dq", "dk", "dv"):
                assert_close(n, to_f64(g[n]), ref[n])
            assert_lse(to_f64(g["lse"]), ref["lse"])
        return desc, check

    def dropout(self):
        B, Hq, Hkv, S, D, causal = self.shape(800)
        p = float(self.rng.choice([0.05, 0.2, 0.5, 0.75]))
        dseed = int(self.rng.integers(0, 1 << 63))
        scale = 1.0 / math.sqrt(D)
        desc = f"dropout B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal={causal} p={p} seed={dseed}"
        x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(self.seed, 2, B, Hq, S, D))

        def check():
            g = run_dropout(x, causal, scale, p, dseed)
            q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
            ref = dr.backward(q, k, v, do, scale, causal, p, dseed)
            for n in ("o", "dq", "dk", "dv"):
                assert_close(n, to_f64(g[n]), ref[n])
            assert_lse(to_f64(g["lse"]), ref["lse"])
        return desc, check

    def rotary(self):
        B, Hq, Hkv, S, D, causal = self.shape(800)
        base = float(self.rng.choice([1e4, 5e5, 1e6]))
        scale = 1.0 / math.sqrt(D)
        desc = f"rope B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal={causal} base={base:g}"
        x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(self.seed, 3, B, Hq, S, D))

        def check():
            g = run_rope(x, causal, scale, base)
            q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
            rnd = rope.backward(q, k, v, do, scale, causal, base, bf16_rotated=True)
            ext = rope.backward(q, k, v, do, scale, causal, base, bf16_rotated=False)
            check_both_readings(g, q, k, rnd, ext, scale, causal, base, Hq // Hkv)
        return desc, check

    def decode(self):
        r = self.rng
        D = int(r.choice([64, 128]))
        Hkv = int(r.choice([1, 2, 4, 8]))
        g = int(r.choice([1, 2, 4, 8, 16]))
        Sq = int(r.choice([s for s in (1, 2, 3, 4, 8, 16) if g * s <= 128]))
        Sk = int(r.integers(Sq, 9000))
        B = int(r.choice([1, 2, 4]))
        causal = bool(r.random() < 0.8)
        scale = 1.0 / math.sqrt(D)
        desc = f"decode B{B} Hq{Hkv * g} Hkv{Hkv} Sq{Sq} Sk{Sk} D{D} causal={causal}"
        x = wl.make_inputs(B, Hkv * g, Hkv, Sk, D, seed=(self.seed, 4, B, g, Sq, Sk, D))

        def check():
            go, gl = run_decode(x, Sq, causal, scale)
            q, k, v = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v"))
            ro, rl = blk.forward_block(q[:, :, Sk - Sq:], k, v, scale, causal, Sk - Sq, 0)
            assert_close("o", go, ro)
            assert_lse(gl, rl)
        return desc, check

    def blocks(self):
        B, Hq, Hkv, S, D, causal = self.shape(1400)
        S = max(S, 4)
        r = self.rng
        nq, nk = int(r.integers(1, 4)), int(r.integers(1, 4))
        qcuts = sorted(set(int(c) for c in r.integers(1, S, nq - 1))) if nq > 1 else []
        kcuts = sorted(set(int(c) for c in r.integers(1, S, nk - 1))) if nk > 1 else []
        scale = 1.0 / math.sqrt(D)
        desc = f"blocks B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal={causal} q{qcuts} k{kcuts}"
        x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(self.seed, 5, B, Hq, S, D))

        def check():
            g = run_blocks(x, causal, scale, qcuts, kcuts)
            q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
            ref = att.backward(q, k, v, do, scale, causal=causal)
            dk_sum, dv_sum = np.zeros_like(k), np.zeros_like(v)
            for q0, q1 in _cuts(S, qcuts):
                for k0, k1 in _cuts(S, kcuts):
                    gdk, gdv = (to_f64(t) for t in g["dkdv"][(q0, k0)])
                    dk_sum[:, :, k0:k1] += gdk
                    dv_sum[:, :, k0:k1] += gdv
                assert_close(f"o[{q0}]", to_f64(g["o"][q0]), ref["o"][:, :, q0:q1])
                assert_lse(to_f64(g["lse"][q0]), ref["lse"][:, :, q0:q1])
                assert_close(f"dq[{q0}]", to_f64(g["dq"][q0]), ref["dq"][:, :, q0:q1])
            # the pieces are rounded to bf16 once per query block before they are summed
            n_q = len(qcuts) + 1
            for n, got in (("dk", dk_sum), ("dv", dv_sum)):
                bound = 2e-2 * n_q + 2.0 ** -10 * float(np.abs(ref[n]).max())
                _assert_close(f"{n} (sum of blocks)", got, ref[n], max_abs=bound)
        return desc, check


def test_random_search():
    s = Search(SEED)
    kinds = [s.plain, s.dropout, s.rotary, s.decode, s.blocks]
    weights = [0.45, 0.15, 0.15, 0.1, 0.15]
    t_end = time.time() + SECONDS
    more = (lambda n: time.time() < t_end) if SECONDS > 0 else (lambda n: n < DEFAULT_CASES)
    n, failures = 0, []
    while more(n):
        desc, check = kinds[int(s.rng.choice(len(kinds), p=weights))]()
        print(f"[case {n}] {desc}", flush=True)
        try:
            check()
        except AssertionError as e:
            failures.append(f"case {n} ({desc}): {e}")
            print(f"FAIL case {n} ({desc}): {e}", flush=True)
        n += 1
    print(f"random search, seed {SEED}: {n} cases, {len(failures)} failures", flush=True)
    assert not failures, "\n".join(failures)
