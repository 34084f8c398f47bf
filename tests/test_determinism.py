"""Bitwise reproducibility on the GPU.

Every output element is written by one thread after a fixed-order reduction
(no atomics; head-subset partials of dK/dV are summed in a fixed order), so
repeated runs, and runs on another stream, must give identical bits. This is
the race detector of the build: a missing barrier or a read of a stage that
is still being written would show up as run-to-run differences.
"""
import numpy as np
import pytest

from gpu_helpers import say, to_dev
from tiled_attention_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 16, 2, 1024, 128),   # several dK/dV head subsets: partials + fixed-order sum
    (1, 8, 8, 777, 64),      # one head per group, ragged tail
    (4, 16, 4, 64, 128),     # short sequences
    (16, 128, 8, 64, 128),   # the batch-16 x 64 workload: one-kernel passes, two head subsets
    (1, 64, 8, 4096, 128),   # the Llama-2-70B layer at 4096 tokens: fp16 products, two head subsets
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_Hq{}_Hkv{}_S{}_D{}".format(*s))
def test_bitwise_repeatable(shape):
    import torch
    import tiled_attention_memory_amd as tam
    B, Hq, Hkv, S, D = shape
    say(f"determinism {shape}")
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(300, S))
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))

    def once(stream=None):
        o, lse = tam.forward(q, k, v, stream=stream)
        dq, dk, dv = tam.backward(q, k, v, o, do, lse, stream=stream)
        torch.cuda.synchronize()
        return [t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else
                t.view(torch.int32).cpu().numpy() for t in (o, lse, dq, dk, dv)]

    first = once()
    for _ in range(3):
        again = once()
        for a, b in zip(first, again):
            assert np.array_equal(a, b)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        other = once(stream=side)
    for a, b in zip(first, other):
        assert np.array_equal(a, b)
