"""GPU parity of the context-parallel building block (include/attn_block.h).

One sequence is cut into query blocks and key/value blocks at their global
positions. Every block pair runs through attn_fwd_block, the parts of a query
block are combined by attn_merge, and the backward protocol (begin, dq per key
block, dq_end, dkdv per key block) produces the gradients. Expected values
come from the fp64 oracles: oracle.blocks for each block pair's partial
results and partial gradients, oracle.attention for the whole sequence.
"""
import math

import numpy as np
import pytest

from gpu_helpers import assert_close, assert_lse, say, to_dev, to_f64
from oracle import attention as att
from oracle import blocks as blk
from tiled_attention_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _cuts(n, cuts):
    e = [0, *cuts, n]
    return [(e[i], e[i + 1]) for i in range(len(e) - 1)]


def _f64(x):
    return att.bf16_bits_to_f64(x)


def _dev_f32(shape):
    import torch
    return torch.empty(shape, dtype=torch.float32, device="cuda")


def run_blocks(x, causal, scale, qcuts, kcuts):
    """Forward (per pair + merge) and the backward protocol on the device."""
    import torch
    import tiled_attention_memory_amd as tam
    B, Hq, S, D = x["q"].shape
    Hkv = x["k"].shape[1]
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    out = {"parts": {}, "o": {}, "lse": {}, "dq": {}, "dkdv": {}}
    kb = _cuts(S, kcuts)
    sk_max = max(k1 - k0 for k0, k1 in kb)
    for q0, q1 in _cuts(S, qcuts):
        Sq = q1 - q0
        qb, dob = q[:, :, q0:q1].contiguous(), do[:, :, q0:q1].contiguous()
        parts = []
        for k0, k1 in kb:
            kk, vv = k[:, :, k0:k1].contiguous(), v[:, :, k0:k1].contiguous()
            o_p, l_p = _dev_f32((B, Hq, Sq, D)), _dev_f32((B, Hq, Sq))
            tam.attn_fwd_block(qb, kk, vv, o_p, l_p, q0, k0, causal=causal, scale=scale)
            parts.append((o_p, l_p))
            out["parts"][(q0, k0)] = (o_p, l_p)
        o = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device="cuda")
        lse = _dev_f32((B, Hq, Sq))
        tam.attn_merge([p[0] for p in parts], [p[1] for p in parts], o, lse)
        out["o"][q0], out["lse"][q0] = o, lse
        ws = torch.empty(tam.attn_bwd_block_workspace_bytes(B, Hq, Hkv, Sq, sk_max, D), dtype=torch.uint8,
                         device="cuda")
        tam.attn_bwd_block_begin(o, dob, lse, ws, Hkv, sk_max)
        for k0, k1 in kb:
            tam.attn_bwd_block_dq(qb, k[:, :, k0:k1].contiguous(), v[:, :, k0:k1].contiguous(), dob, ws, q0, k0,
                                  causal=causal, scale=scale)
        dq = torch.empty_like(qb)
        tam.attn_bwd_block_dq_end(dq, ws, Hkv, sk_max, scale=scale)
        out["dq"][q0] = dq
        for k0, k1 in kb:
            kk, vv = k[:, :, k0:k1].contiguous(), v[:, :, k0:k1].contiguous()
            dk, dv = torch.empty_like(kk), torch.empty_like(vv)
            tam.attn_bwd_block_dkdv(qb, kk, vv, dob, dk, dv, ws, q0, k0, causal=causal, scale=scale)
            out["dkdv"][(q0, k0)] = (dk, dv)
    torch.cuda.synchronize()
    return out


CASES = [
    # B, Hq, Hkv, S, D, causal, query cuts, key cuts; key blocks of 1024 keys
    # or more take the fp16 dK/dV kernel (the last two cases)
    (1, 4, 2, 700, 128, True, [300], [256, 500]),
    (1, 8, 1, 333, 128, True, [64, 200], [100]),
    (2, 4, 4, 257, 64, True, [129], [64, 190]),
    (1, 4, 2, 300, 128, False, [111], [150]),
    # query blocks of 30 and 60 rows: 4 and 2 query heads per unit
    (1, 8, 2, 90, 128, True, [30], [40]),
    (1, 4, 2, 2200, 128, True, [1000], [1100]),
    (1, 2, 1, 2100, 64, False, [900], [1030]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_S{c[3]}_D{c[4]}_"
                         f"{'causal' if c[5] else 'full'}_q{c[6]}_k{c[7]}")
def test_blocks_against_oracles(case):
    B, Hq, Hkv, S, D, causal, qcuts, kcuts = case
    say(f"blocks {case}")
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(300, S, D, int(causal)))
    scale = 1.0 / math.sqrt(D)
    g = run_blocks(x, causal, scale, qcuts, kcuts)
    q, k, v, do = (_f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = att.backward(q, k, v, do, scale, causal=causal)
    dk_sum, dv_sum = np.zeros_like(k), np.zeros_like(v)
    for q0, q1 in _cuts(S, qcuts):
        for k0, k1 in _cuts(S, kcuts):
            # partial results of the pair: rows with no visible key are exactly 0 / -inf
            po, pl = blk.forward_block(q[:, :, q0:q1], k[:, :, k0:k1], v[:, :, k0:k1], scale, causal, q0, k0)
            go, gl = (to_f64(t) for t in g["parts"][(q0, k0)])
            empty = np.isneginf(pl)
            assert np.array_equal(np.isneginf(gl), empty), "rows without keys differ"
            assert np.all(go[empty] == 0.0)
            if (~empty).any():
                assert_close(f"o_part[{q0},{k0}]", go[~empty], po[~empty])
                assert_lse(gl[~empty], pl[~empty])
            # this pair's dK, dV from the merged o, lse of the oracle
            pg = blk.backward_block(q[:, :, q0:q1], k[:, :, k0:k1], v[:, :, k0:k1], ref["o"][:, :, q0:q1],
                                    do[:, :, q0:q1], ref["lse"][:, :, q0:q1], scale, causal, q0, k0)
            gdk, gdv = (to_f64(t) for t in g["dkdv"][(q0, k0)])
            assert_close(f"dk[{q0},{k0}]", gdk, pg["dk"])
            assert_close(f"dv[{q0},{k0}]", gdv, pg["dv"])
            dk_sum[:, :, k0:k1] += gdk
            dv_sum[:, :, k0:k1] += gdv
        assert_close(f"o[{q0}]", to_f64(g["o"][q0]), ref["o"][:, :, q0:q1])
        assert_lse(to_f64(g["lse"][q0]), ref["lse"][:, :, q0:q1])
        assert_close(f"dq[{q0}]", to_f64(g["dq"][q0]), ref["dq"][:, :, q0:q1])
    # the pieces add up to the whole-sequence gradients (sum of bf16 pieces: one
    # extra rounding per piece)
    n_q = len(qcuts) + 1
    assert_close("dk (sum of blocks)", dk_sum, ref["dk"], max_abs=2e-2 * n_q)
    assert_close("dv (sum of blocks)", dv_sum, ref["dv"], max_abs=2e-2 * n_q)


def test_hidden_block_and_offsets_past_the_ends():
    """Keys entirely after the queries, and offsets far outside [-Sq, Sk]."""
    import torch
    import tiled_attention_memory_amd as tam
    say("fully hidden block, far offsets")
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 1, 70, 90, 128
    x = wl.make_inputs(B, Hq, Hkv, 160, D, seed=(301,))
    q = to_dev(x["q"][:, :, :Sq])
    k, v = to_dev(x["k"][:, :, :Sk]), to_dev(x["v"][:, :, :Sk])
    o_p, l_p = _dev_f32((B, Hq, Sq, D)), _dev_f32((B, Hq, Sq))
    tam.attn_fwd_block(q, k, v, o_p, l_p, 0, Sq, causal=True)          # keys start after the last query
    assert torch.all(o_p == 0) and torch.all(torch.isneginf(l_p))
    tam.attn_fwd_block(q, k, v, o_p, l_p, 0, 1 << 40, causal=True)     # far in the future
    assert torch.all(o_p == 0) and torch.all(torch.isneginf(l_p))
    tam.attn_fwd_block(q, k, v, o_p, l_p, 1 << 40, 0, causal=True)     # far in the past: all keys visible
    full_o, full_l = _dev_f32((B, Hq, Sq, D)), _dev_f32((B, Hq, Sq))
    tam.attn_fwd_block(q, k, v, full_o, full_l, 0, 0, causal=False)
    torch.cuda.synchronize()
    # same arithmetic through the causal and the unmasked kernel
    assert float((o_p - full_o).abs().max()) <= 1e-6 and float((l_p - full_l).abs().max()) <= 1e-6


def test_single_block_matches_attn_fwd_bitwise():
    """One block at offset 0 merged alone reproduces attn_fwd exactly."""
    import torch
    import tiled_attention_memory_amd as tam
    say("single block vs attn_fwd")
    B, Hq, Hkv, S, D = 1, 8, 2, 321, 128
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(302,))
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o_ref, l_ref = tam.forward(q, k, v, causal=True)
    o_p, l_p = _dev_f32((B, Hq, S, D)), _dev_f32((B, Hq, S))
    tam.attn_fwd_block(q, k, v, o_p, l_p, 0, 0, causal=True)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    tam.attn_merge([o_p], [l_p], o, lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)


def test_context_parallel_rank_at_full_size():
    """The last of 8 ranks of the 81920-token workload: its 10240 query rows against
    all 8 key blocks, forward (8 block calls + merge) and the backward protocol.

    O, LSE and dQ of sampled rows against the whole-sequence oracle (a row's
    results depend on its own score row only); dK and dV, summed over the key
    blocks, through two exact properties of this query block's contribution:
    sum_j dK_j = 0 (shifting every key leaves its outputs unchanged) and
    sum_j dV_j = sum over its rows and the group's heads of dO.
    """
    import torch
    import tiled_attention_memory_amd as tam
    w = wl.BY_NAME["very_long_s81920"]
    n = 8
    s = w.S // n
    r = n - 1
    say(f"context-parallel rank {r} of {n}, {w.name}")
    x = wl.workload_inputs(w)
    q, k, v, do = (to_dev(x[nm]) for nm in ("q", "k", "v", "do"))
    q0 = r * s
    qb, dob = q[:, :, q0:q0 + s].contiguous(), do[:, :, q0:q0 + s].contiguous()
    kbs = [(k[:, :, b * s:(b + 1) * s].contiguous(), v[:, :, b * s:(b + 1) * s].contiguous()) for b in range(n)]
    parts = []
    for b, (kk, vv) in enumerate(kbs):
        o_p, l_p = _dev_f32((w.B, w.Hq, s, w.D)), _dev_f32((w.B, w.Hq, s))
        tam.attn_fwd_block(qb, kk, vv, o_p, l_p, q0, b * s, causal=True, scale=w.scale)
        parts.append((o_p, l_p))
    o = torch.empty_like(qb)
    lse = _dev_f32((w.B, w.Hq, s))
    tam.attn_merge([p[0] for p in parts], [p[1] for p in parts], o, lse)
    ws = torch.empty(tam.attn_bwd_block_workspace_bytes(w.B, w.Hq, w.Hkv, s, s, w.D), dtype=torch.uint8,
                     device="cuda")
    tam.attn_bwd_block_begin(o, dob, lse, ws, w.Hkv, s)
    for b, (kk, vv) in enumerate(kbs):
        tam.attn_bwd_block_dq(qb, kk, vv, dob, ws, q0, b * s, causal=True, scale=w.scale)
    dq = torch.empty_like(qb)
    tam.attn_bwd_block_dq_end(dq, ws, w.Hkv, s, scale=w.scale)
    dk_sum = torch.zeros((w.B, w.Hkv, w.D), dtype=torch.float64, device="cuda")
    dv_sum = torch.zeros_like(dk_sum)
    for b, (kk, vv) in enumerate(kbs):
        dk, dv = torch.empty_like(kk), torch.empty_like(vv)
        tam.attn_bwd_block_dkdv(qb, kk, vv, dob, dk, dv, ws, q0, b * s, causal=True, scale=w.scale)
        dk_sum += dk.double().sum(dim=2)
        dv_sum += dv.double().sum(dim=2)
    torch.cuda.synchronize()
    say("oracle on sampled rows")
    qh, kh, vh, doh = (_f64(x[nm]) for nm in ("q", "k", "v", "do"))
    rng = np.random.default_rng(7)
    rows = np.concatenate([np.arange(0, 64), np.arange(s - 64, s), rng.choice(s, 64, replace=False)])
    go, gl, gq = to_f64(o), to_f64(lse), to_f64(dq)
    for h in (0, 5):
        ref = att.rows_forward_backward(qh[0, h], kh[0, 0], vh[0, 0], doh[0, h], q0 + rows, w.scale)
        assert_close(f"o rows h{h}", go[0, h, rows], ref["o"])
        assert_lse(gl[0, h, rows], ref["lse"])
        assert_close(f"dq rows h{h}", gq[0, h, rows], ref["dq"])
    dk_sum, dv_sum = dk_sum.cpu().numpy(), dv_sum.cpu().numpy()
    do_sum = doh[:, :, q0:q0 + s].reshape(w.B, w.Hkv, w.group, s, w.D).sum(axis=(2, 3))
    tol = 2e-2 * math.sqrt(w.S)
    assert np.max(np.abs(dk_sum)) <= tol, np.max(np.abs(dk_sum))
    assert np.max(np.abs(dv_sum - do_sum)) <= tol, np.max(np.abs(dv_sum - do_sum))
