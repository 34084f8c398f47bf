"""GPU parity of attention with dropout (include/attn_dropout.h).

The keep mask is integer work and is compared bit for bit: with Q = 0 every
visible key of row i has probability 1/(i+1), and with V the identity (V_j =
e_j) the output row i is the row of the mask times r/(i+1), so the zero
pattern of O is the mask. Outputs and gradients are compared element by element
with the dropout oracle (oracle.dropout), which draws the same Philox bytes.
"""
import math

import numpy as np
import pytest

from gpu_helpers import assert_close, assert_lse, say, to_dev, to_f64
from oracle import attention as att
from oracle import dropout as dr
from tiled_attention_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu


def run(x, causal, scale, p, seed):
    import torch
    import tiled_attention_memory_amd as tam
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    B, Hq, S, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    tam.attn_fwd_dropout(q, k, v, o, lse, p, seed, causal=causal, scale=scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    tam.attn_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, tam.workspace_for(q, k), p, seed, causal=causal,
                         scale=scale)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("p,seed", [(0.5, 0), (0.1, 123456789), (0.9, (1 << 63) + 12345)])
def test_mask_is_bit_exact(p, seed):
    import torch
    say(f"dropout mask p={p} seed={seed}")
    B, Hq, Hkv, S, D = 2, 4, 2, 128, 128
    bits = lambda a: np.ascontiguousarray(a.astype(np.float32)).view(np.uint32).__rshift__(16).astype(np.uint16)
    x = {"q": bits(np.zeros((B, Hq, S, D))), "k": wl.make_inputs(B, Hq, Hkv, S, D, seed=(410,))["k"],
         "v": bits(np.broadcast_to(np.eye(S, D), (B, Hkv, S, D))), "do": bits(np.zeros((B, Hq, S, D)))}
    g = run(x, True, 0.125, p, seed)
    o = to_f64(g["o"])
    r = dr.rescale(p)
    for b in range(B):
        for h in range(Hq):
            m = dr.keep_mask(b, h, Hq, np.arange(S), np.arange(S), p, seed)
            vis = np.tril(np.ones((S, S), dtype=bool))
            got = o[b, h] != 0
            assert np.array_equal(got & vis, m & vis), f"mask differs at b={b} h={h}"
            assert not np.any(got & ~vis)
            want = np.where(m & vis, r / (np.arange(S)[:, None] + 1), 0.0)
            # kept values: r/(i+1) rounded to bf16 once for the product with V and once on output
            assert np.all(np.abs(o[b, h] - want) <= 2.0 ** -7 * want)


CASES = [
    # B, Hq, Hkv, S, D, causal, p; up to 511 keys the backward runs the bf16
    # hi + lo gradient products, from 512 the fp16 ones with the dropout scale
    # folded into the power-of-two operand scales (p = 0.75: r = 4 = 2^2)
    (1, 4, 2, 200, 128, True, 0.1),
    (2, 8, 2, 333, 128, True, 0.5),
    (1, 4, 4, 129, 64, True, 0.25),
    (1, 6, 2, 190, 128, False, 0.3),
    (1, 4, 2, 640, 128, True, 0.1),
    (1, 4, 1, 600, 64, True, 0.5),
    (1, 2, 2, 530, 128, False, 0.3),
    (1, 2, 1, 520, 128, True, 0.75),
    # short sequences: 2 and 4 query heads per unit of the forward and dQ kernels
    (2, 8, 2, 50, 128, True, 0.2),
    (1, 8, 2, 24, 64, False, 0.4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_S{}_D{}_{}_p{}".format(
    *c[:5], "causal" if c[5] else "full", c[6]))
def test_dropout_against_oracle(case):
    B, Hq, Hkv, S, D, causal, p = case
    seed = 0x5EED0000 + S
    say(f"dropout {case}")
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(411, S, D))
    scale = 1.0 / math.sqrt(D)
    g = run(x, causal, scale, p, seed)
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = dr.backward(q, k, v, do, scale, causal, p, seed)
    for name in ("o", "dq", "dk", "dv"):
        assert_close(name, to_f64(g[name]), ref[name])
    assert_lse(to_f64(g["lse"]), ref["lse"])


def test_smoke_workload_with_dropout():
    w = wl.BY_NAME["smoke_s256_d64"]
    say("dropout on the smoke workload")
    x = wl.workload_inputs(w)
    g = run(x, True, w.scale, 0.1, 2024)
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = dr.backward(q, k, v, do, w.scale, True, 0.1, 2024)
    for name in ("o", "dq", "dk", "dv"):
        assert_close(name, to_f64(g[name]), ref[name])


def test_zero_probability_is_plain_attention_and_seeds_matter():
    import torch
    import tiled_attention_memory_amd as tam
    say("dropout p below 1/512, and seed dependence")
    B, Hq, Hkv, S, D = 1, 4, 2, 256, 128
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(412,))
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o_ref, l_ref = tam.forward(q, k, v)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    tam.attn_fwd_dropout(q, k, v, o, lse, 0.001, 99)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref)
    o1, o2 = torch.empty_like(o_ref), torch.empty_like(o_ref)
    tam.attn_fwd_dropout(q, k, v, o1, lse, 0.2, 1)
    tam.attn_fwd_dropout(q, k, v, o2, lse, 0.2, 1)
    tam.attn_fwd_dropout(q, k, v, o, lse, 0.2, 2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert not torch.equal(o1.view(torch.int16), o.view(torch.int16))


def test_llama2_layer_heads_with_dropout():
    """S=4096, 64/8 heads, p = 0.1 (the fp16 backward): every element of O, LSE and
    dQ for two query heads of kv head 3; dK and dV need all eight heads of the
    group and are covered at this size without dropout in test_parity.py and
    with dropout over 512 keys above."""
    w = wl.BY_NAME["llama2_70b_layer_s4096"]
    p, seed, kvh = 0.1, 77, 3
    heads = [kvh * w.group + 1, kvh * w.group + 6]
    say(f"workload {w.name} with dropout p={p}: heads {heads}")
    x = wl.workload_inputs(w)
    g = run(x, True, w.scale, p, seed)
    q, do = (att.bf16_bits_to_f64(x[n][:, heads]) for n in ("q", "do"))
    k, v = (att.bf16_bits_to_f64(x[n][:, kvh:kvh + 1]) for n in ("k", "v"))
    rows = np.arange(w.S)
    say("oracle on the two heads")
    ref = dr.backward(q, k, v, do, w.scale, True, p, seed,
                      masks=lambda b, h: dr.keep_mask(b, heads[h], w.Hq, rows, rows, p, seed))
    for name in ("o", "dq"):
        assert_close(name, to_f64(g[name])[:, heads], ref[name])
    assert_lse(to_f64(g["lse"])[:, heads], ref["lse"])
