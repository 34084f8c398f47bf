"""GPU parity of attention with rotary position embedding (include/attn_rope.h).

Expected values come from oracle.rope: fp64 rotation with the rotated Q and K
rounded to bf16 (the precision of the attention inputs), the plain attention
oracle on the rotated pair, gradients rotated back. The same outputs are also
held against the plain fp64 rotation with no rounding of the rotated pair:
O, dQ, dK and dV at the same tolerances, and the LSE at 1e-3 beyond the
amount that rounding the rotated pair to bf16 moves it. That amount has a
closed bound: the LSE of a row is 1-Lipschitz in the largest change of its
scores, so it moves by at most max_j |s~_ij - s_ij|, the largest change the
rounding makes to one of the row's visible scores (computed here exactly).
"""
import math

import numpy as np
import pytest

from gpu_helpers import assert_close, assert_lse, say, to_dev, to_f64
from oracle import attention as att
from oracle import rope
from tiled_attention_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu


def run(x, causal, scale, base):
    import torch
    import tiled_attention_memory_amd as tam
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    B, Hq, S, D = q.shape
    ws = tam.rope_workspace_for(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    tam.attn_fwd_rope(q, k, v, o, lse, ws, base, causal=causal, scale=scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    tam.attn_bwd_rope(q, k, v, o, do, lse, dq, dk, dv, ws, base, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


CASES = [
    # B, Hq, Hkv, S, D, causal, base
    (1, 4, 2, 300, 128, True, 1e4),
    (1, 8, 1, 1000, 128, True, 1e6),
    (2, 4, 4, 129, 64, True, 1e4),
    (1, 6, 2, 190, 128, False, 5e5),
    (2, 8, 2, 40, 128, True, 1e4),   # 2 query heads per unit
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_S{}_D{}_{}_base{:g}".format(
    *c[:5], "causal" if c[5] else "full", c[6]))
def test_rope_against_oracle(case):
    B, Hq, Hkv, S, D, causal, base = case
    say(f"rope {case}")
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(420, S, D))
    scale = 1.0 / math.sqrt(D)
    g = run(x, causal, scale, base)
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    rnd = rope.backward(q, k, v, do, scale, causal, base, bf16_rotated=True)
    ext = rope.backward(q, k, v, do, scale, causal, base, bf16_rotated=False)
    for ref, what in ((rnd, "rounded to bf16"), (ext, "in fp64")):
        print(f"  against the oracle with the rotated pair {what}")
        for name in ("o", "dq", "dk", "dv"):
            assert_close(name, to_f64(g[name]), ref[name])
        allowance = None if ref is rnd else lse_rounding_allowance(rnd, ext, scale, causal, Hq // Hkv)
        assert_lse(to_f64(g["lse"]), ref["lse"], allowance)


def lse_rounding_allowance(rnd, ext, scale, causal, group):
    """max_j |s~_ij - s_ij| per row: how far rounding the rotated pair moves each score row."""
    qr, kr = rnd["q_rot"], np.repeat(rnd["k_rot"], group, axis=1)
    qe, ke = ext["q_rot"], np.repeat(ext["k_rot"], group, axis=1)
    ds = np.abs(scale * (qr @ np.swapaxes(kr, -1, -2) - qe @ np.swapaxes(ke, -1, -2)))
    if causal:
        S = ds.shape[-1]
        ds = np.where(np.arange(S)[None, :] <= np.arange(S)[:, None], ds, 0.0)
    return ds.max(axis=-1)


def test_rope_at_long_positions_sampled():
    """Positions up to 32767 (the 32k-context workload's shape, one kv group): the fp64
    angles keep the rotation accurate far from the start; sampled rows against the oracle."""
    import torch
    import tiled_attention_memory_amd as tam
    w = wl.BY_NAME["long_context_s32768_k3"]
    say("rope at 32k positions, base 1e6")
    B, Hq, Hkv, S, D = 1, 4, 1, w.S, w.D
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(421,), k_mult=3.0)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    ws = tam.rope_workspace_for(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    tam.attn_fwd_rope(q, k, v, o, lse, ws, 1e6, scale=w.scale)
    torch.cuda.synchronize()
    qh, kh, vh = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v"))
    pos = np.arange(S)
    rows = np.concatenate([np.arange(0, 32), np.arange(S - 64, S), np.random.default_rng(5).choice(S, 32)])
    go, gl = to_f64(o), to_f64(lse)
    vis = np.arange(S)[None, :] <= rows[:, None]
    ke = rope.rotate(kh[0, 0], pos, 1e6)
    kr = rope.round_bf16(ke)
    for h in (0, 3):
        qe = rope.rotate(qh[0, h][rows], rows, 1e6)
        qr = rope.round_bf16(qe)
        s_r, s_e = w.scale * (qr @ kr.T), w.scale * (qe @ ke.T)
        allowance = np.where(vis, np.abs(s_r - s_e), 0.0).max(axis=1)
        for s, what, allow in ((s_r, "bf16", None), (s_e, "fp64", allowance)):
            p, l = att.softmax_rows(np.where(vis, s, -np.inf))
            assert_close(f"o rows h{h} ({what} rotation)", go[0, h, rows], p @ vh[0, 0])
            assert_lse(gl[0, h, rows], l, allow)
