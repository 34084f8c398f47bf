"""GPU parity of attention with rotary position embedding (include/attn_rope.h).

Expected values come from oracle.rope: fp64 rotation with the rotated Q and K
rounded to bf16 (the precision of the attention inputs), the plain attention
oracle on the rotated pair, gradients rotated back. This is the parity
reading.

The kernels evaluate the rotation in fp32 with an fp32 (cos, sin) table. That
result lies within 2^-22 (|x_d| + |x_{d+D/2}|) of the exact rotation, so a
rotated value whose exact value lies that close to a bf16 rounding midpoint
may be rounded to the other bf16 neighbour (about one value in 60 000; a
seeded random search found LSE errors of 1.03-2.23e-3 from it without an
allowance). The LSE, held at 1e-3, gets an allowance for exactly those
values: the largest change of a visible score that turning each of them to
its other neighbour can make (the LSE of a row is 1-Lipschitz in the largest
change of its scores). O, dQ, dK and dV need none at their 2e-2.

The same outputs are also held against the plain fp64 rotation with no
rounding of the rotated pair. Rounding the rotated inputs moves the exact
result itself, by an amount the two oracle readings give per element: O, dQ,
dK and dV are held to the same tolerances beyond that amount, and the LSE
beyond the largest change the rounding makes to one of the row's visible
scores (plus the allowance above). Without these allowances the search found
dK and dV up to 2.16e-2 beyond the output rounding: the effect of the bf16
inputs, not of the kernels.
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
    # B, Hq, Hkv, S, D, causal, base, input seed
    (1, 4, 2, 300, 128, True, 1e4, (420, 300, 128)),
    (1, 8, 1, 1000, 128, True, 1e6, (420, 1000, 128)),
    (2, 4, 4, 129, 64, True, 1e4, (420, 129, 64)),
    (1, 6, 2, 190, 128, False, 5e5, (420, 190, 128)),
    (2, 8, 2, 40, 128, True, 1e4, (420, 40, 128)),   # 2 query heads per unit
    # inputs where the fp32 rotation rounds some rotated values to the other
    # bf16 neighbour (LSE 2.2e-3 off the rounded reading without the
    # allowance), and where the unrounded reading differs most (dV 2.07e-2
    # beyond the output rounding without its allowance)
    (3, 12, 2, 691, 64, True, 5e5, (778, 3, 3, 12, 691, 64)),
    (3, 16, 1, 256, 128, True, 1e4, (778, 3, 3, 16, 256, 128)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_S{}_D{}_{}_base{:g}".format(
    *c[:5], "causal" if c[5] else "full", c[6]))
def test_rope_against_oracle(case):
    B, Hq, Hkv, S, D, causal, base, seed = case
    say(f"rope {case}")
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=seed)
    scale = 1.0 / math.sqrt(D)
    g = run(x, causal, scale, base)
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    rnd = rope.backward(q, k, v, do, scale, causal, base, bf16_rotated=True)
    ext = rope.backward(q, k, v, do, scale, causal, base, bf16_rotated=False)
    check_both_readings(g, q, k, rnd, ext, scale, causal, base, Hq // Hkv)


def check_both_readings(g, q, k, rnd, ext, scale, causal, base, group):
    amb = ambiguity_allowance(q, k, rnd, scale, causal, base, group)
    print("  against the oracle with the rotated pair rounded to bf16")
    for name in ("o", "dq", "dk", "dv"):
        assert_close(name, to_f64(g[name]), rnd[name])
    assert_lse(to_f64(g["lse"]), rnd["lse"], amb)
    print("  against the oracle with the rotated pair in fp64, beyond what the rounding moves")
    for name in ("o", "dq", "dk", "dv"):
        assert_close(name, to_f64(g[name]), ext[name], allowance=np.abs(rnd[name] - ext[name]))
    assert_lse(to_f64(g["lse"]), ext["lse"], lse_rounding_allowance(rnd, ext, scale, causal, group) + amb)


def other_neighbour_step(x, rotated_exact):
    """Per element of a rotated [..., S, D] tensor: |other bf16 neighbour - rounded value| where the
    kernels' fp32 rotation may round to the other neighbour (its exact value within 2^-22 (|x_d| +
    |x_{d+D/2}|) of a bf16 rounding midpoint), 0 elsewhere."""
    D = x.shape[-1]
    e = 2.0 ** -22 * (np.abs(x[..., : D // 2]) + np.abs(x[..., D // 2:]))
    e = np.concatenate([e, e], axis=-1)
    _, ex = np.frexp(rotated_exact)
    unit = np.ldexp(1.0, ex - 8)                    # bf16 spacing in the value's binade
    t = rotated_exact / unit
    near = np.abs(t - (np.floor(t) + 0.5)) * unit <= e
    return np.where(near & (rotated_exact != 0), unit, 0.0)


def ambiguity_allowance(q, k, rnd, scale, causal, base, group):
    """Per row: the largest change of a visible score if every value of the rounded rotated pair that
    the kernels may round the other way did so."""
    S = q.shape[2]
    pos = np.arange(S)
    dq = other_neighbour_step(q, rope.rotate(q, pos, base))
    dk = np.repeat(other_neighbour_step(k, rope.rotate(k, pos, base)), group, axis=1)
    qr, kr = np.abs(rnd["q_rot"]), np.abs(np.repeat(rnd["k_rot"], group, axis=1))
    kt = lambda a: np.swapaxes(a, -1, -2)
    ds = abs(scale) * (dq @ kt(kr) + qr @ kt(dk) + dq @ kt(dk))
    if causal:
        ds = np.where(np.arange(S)[None, :] <= np.arange(S)[:, None], ds, 0.0)
    return ds.max(axis=-1)


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
