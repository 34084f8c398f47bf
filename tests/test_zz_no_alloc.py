"""attn_bwd_noalloc (the backward pass on the library's fixed scratch) against attn_bwd.

Calls in a row on the same GPU, the second with a smaller input, so later
calls run on a scratch that still holds an earlier call's contents; the third
is a batch of 64-token sequences, whose one-kernel backward keeps its dK/dV
partials at the start of the scratch. Each is compared with attn_bwd on a
caller workspace (the same kernels: the outputs must be bitwise equal), and
the smaller ones also with the fp64 oracle. Sizes whose workspace exceeds the
scratch are rejected before anything runs.
"""
import math

import numpy as np
import pytest

from gpu_helpers import assert_close, say, to_dev, to_f64
from oracle import attention as att
from tiled_attention_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _run_both(x, causal, scale):
    import torch
    import tiled_attention_memory_amd as tam
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = tam.forward(q, k, v, causal=causal, scale=scale)
    want = tam.backward(q, k, v, o, do, lse, causal=causal, scale=scale)
    got = [torch.empty_like(t) for t in want]
    # poison the outputs: every element must be written
    for t in got:
        t.view(torch.int16).fill_(0x7fc1)
    tam.attn_bwd_noalloc(q, k, v, o, do, lse, *got, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return got, want


def test_noalloc_matches_attn_bwd_on_two_calls():
    import torch
    import tiled_attention_memory_amd as tam
    cases = [  # B, Hq, Hkv, S, D, causal; the first is the Llama-2-70B layer shape (202 MiB of workspace)
        (1, 64, 8, 4096, 128, True),
        (1, 8, 2, 1000, 128, True),
        (16, 32, 4, 64, 128, True),   # one-kernel backward with 4 head subsets of partials
    ]
    need = [tam.attn_bwd_workspace_bytes(*c[:5]) for c in cases]
    assert need[1] < need[0] <= tam.NOALLOC_SCRATCH_BYTES
    for i, (B, Hq, Hkv, S, D, causal) in enumerate(cases):
        say(f"noalloc call {i}: {(B, Hq, Hkv, S, D, causal)}")
        x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(700, i))
        scale = 1.0 / math.sqrt(D)
        got, want = _run_both(x, causal, scale)
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            same = torch.equal(g.view(torch.int16), w.view(torch.int16))
            print(f"    {name}: bitwise equal to attn_bwd: {same}", flush=True)
            assert same, name
        if i >= 1:
            q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
            ref = att.backward(q, k, v, do, scale, causal=causal)
            for name, g in zip(("dq", "dk", "dv"), got):
                assert_close(name, to_f64(g), ref[name])


def test_noalloc_rejects_sizes_beyond_the_scratch():
    import torch
    import tiled_attention_memory_amd as tam
    B, Hq, Hkv, S, D = 1, 32, 8, 32768, 128      # 584 MiB of workspace
    assert tam.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D) > tam.NOALLOC_SCRATCH_BYTES
    bf = torch.bfloat16
    q = torch.zeros((B, Hq, S, D), dtype=bf, device="cuda")
    k = torch.zeros((B, Hkv, S, D), dtype=bf, device="cuda")
    lse = torch.zeros((B, Hq, S), dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)]
    with pytest.raises(tam.AttnError) as e:
        tam.attn_bwd_noalloc(q, k, k.clone(), q.clone(), q.clone(), lse, *outs)
    assert e.value.status == 10
