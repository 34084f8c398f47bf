"""CPU checks of the dropout oracle (oracle.dropout): its generator against published
known answers, its attention against the plain oracle and torch, its mask statistics,
and planted mistakes that these checks must catch."""
import inspect
import math
import os
import types

import numpy as np
import pytest

from oracle import attention as att
from oracle import dropout as dr
from oracle_pins import close, rand

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def kat_rows():
    rows = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            rows.append([int(x, 16) for x in line.split()])
    return rows


def pin_philox_kat(mod):
    ok = True
    for r in kat_rows():
        out = mod.philox4x32_10(*r[:4], r[4], r[5])
        ok &= [int(x) for x in out] == r[6:]
    return ok


def pin_zero_p_is_plain_attention(mod):
    B, hq, hkv, S, D = 1, 4, 2, 19, 8
    q, k, v, do = rand((B, hq, S, D), 61), rand((B, hkv, S, D), 62), rand((B, hkv, S, D), 63), rand((B, hq, S, D), 64)
    ok = True
    for causal in (True, False):
        a = mod.backward(q, k, v, do, 0.3, causal, 0.0, 12345)
        b = att.backward(q, k, v, do, 0.3, causal=causal)
        ok &= all(close(a[n], b[n], 1e-12) for n in ("o", "lse", "dq", "dk", "dv"))
    return ok


def pin_explicit_mask_against_torch(mod):
    """With a given mask, forward and gradients equal torch autograd of (softmax(S) * M * r) V."""
    import torch
    B, hq, hkv, S, D = 1, 4, 2, 13, 8
    q, k, v, do = rand((B, hq, S, D), 71), rand((B, hkv, S, D), 72), rand((B, hkv, S, D), 73), rand((B, hq, S, D), 74)
    rng = np.random.default_rng(75)
    masks = rng.random((B, hq, S, S)) > 0.3
    p = 0.3
    r = mod.rescale(p)
    ok = True
    for causal in (True, False):
        a = mod.backward(q, k, v, do, 0.5, causal, p, 0, masks=lambda b, h: masks[b, h])
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        kr, vr = tk.repeat_interleave(hq // hkv, dim=1), tv.repeat_interleave(hq // hkv, dim=1)
        s = 0.5 * torch.matmul(tq, kr.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1) * torch.tensor(masks) * r, vr)
        o.backward(torch.tensor(do))
        ok &= close(a["o"], o.detach().numpy(), 1e-12) and close(a["dq"], tq.grad.numpy(), 1e-11)
        ok &= close(a["dk"], tk.grad.numpy(), 1e-11) and close(a["dv"], tv.grad.numpy(), 1e-11)
        ok &= close(a["lse"], torch.logsumexp(s, dim=-1).detach().numpy(), 1e-12)
    return ok


def pin_keep_rate_and_layout(mod):
    """Keep fraction 1 - t/256 within 5 sigma; sub-blocks of the mask are blocks of the whole mask;
    different heads and seeds give different masks."""
    ok = True
    for p in (0.1, 0.5, 0.9):
        m = mod.keep_mask(1, 3, 8, np.arange(512), np.arange(512), p, 987654321)
        q_keep = 1 - mod.threshold(p) / 256
        n = m.size
        ok &= abs(m.mean() - q_keep) <= 5 * math.sqrt(q_keep * (1 - q_keep) / n)
        sub = mod.keep_mask(1, 3, 8, np.arange(100, 140), np.arange(37, 301), p, 987654321)
        ok &= bool(np.array_equal(sub, m[100:140, 37:301]))
    a = mod.keep_mask(0, 0, 4, np.arange(64), np.arange(64), 0.5, 1)
    ok &= not np.array_equal(a, mod.keep_mask(0, 1, 4, np.arange(64), np.arange(64), 0.5, 1))
    ok &= not np.array_equal(a, mod.keep_mask(0, 0, 4, np.arange(64), np.arange(64), 0.5, 2))
    ok &= not np.array_equal(a, mod.keep_mask(1, 0, 4, np.arange(64), np.arange(64), 0.5, 1))
    return ok


def pin_finite_differences(mod):
    """Gradients of L = sum(O * dO) for a fixed generated mask, by central differences."""
    B, hq, hkv, S, D = 1, 2, 1, 6, 4
    q, k, v, do = rand((B, hq, S, D), 81), rand((B, hkv, S, D), 82), rand((B, hkv, S, D), 83), rand((B, hq, S, D), 84)
    p, seed, eps = 0.4, 77, 1e-6
    g = mod.backward(q, k, v, do, 0.7, True, p, seed)
    ok = True
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name[1]] = xp
            lp = (mod.backward(args["q"], args["k"], args["v"], do, 0.7, True, p, seed)["o"] * do).sum()
            args[name[1]] = xm
            lm = (mod.backward(args["q"], args["k"], args["v"], do, 0.7, True, p, seed)["o"] * do).sum()
            num[idx] = (lp - lm) / (2 * eps)
        ok &= float(np.max(np.abs(num - g[name]))) <= 1e-6 * max(1.0, float(np.max(np.abs(num))))
    return ok


def pin_mask_hand_block(mod):
    """The 4 x 4 block at rows 0..3, keys 0..3 of batch 0, head 0 with seed 0 has counter and key 0,
    so its bytes are those of the first known answer: row i reads word i, key j byte j (low byte
    first): d5 e8 27 66 / 8d c5 69 e1 / 4c ac 57 bc / d8 db 00 9b. At p = 1/2 (t = 128) a pair is
    kept when its byte is at least 0x80."""
    want = np.array([[1, 1, 0, 0], [1, 1, 0, 1], [0, 1, 0, 1], [1, 1, 0, 1]], dtype=bool)
    m = mod.keep_mask(0, 0, 4, np.arange(4), np.arange(4), 0.5, 0)
    return bool(np.array_equal(m, want)) and mod.threshold(0.5) == 128 and mod.rescale(0.5) == 2.0


ALL = [pin_philox_kat, pin_mask_hand_block, pin_zero_p_is_plain_attention, pin_explicit_mask_against_torch, pin_keep_rate_and_layout,
       pin_finite_differences]


@pytest.mark.parametrize("pin", ALL, ids=lambda p: p.__name__)
def test_dropout_pin(pin):
    assert pin(dr)


SOURCE = inspect.getsource(dr)
MUTATIONS = {
    "philox_swapped_multipliers": ("M0, M1 = 0xD2511F53, 0xCD9E8D57", "M0, M1 = 0xCD9E8D57, 0xD2511F53"),
    "philox_no_key_schedule": ("k0 = (k0 + np.uint64(W0)) & MASK32", "k0 = k0"),
    "mask_byte_from_row": ("(np.uint64(8) * (cols % np.uint64(4)))", "(np.uint64(8) * (cols % np.uint64(2)))"),
    "keep_below_threshold": ("return byte >= np.uint64(t)", "return byte < np.uint64(256 - t)"),
    "no_rescale": ("pd = p * mask * r", "pd = p * mask"),
    "ds_without_mask": ("ds = p * (mask * r * dpd - delta[:, None])", "ds = p * (dpd - delta[:, None])"),
    "delta_from_undropped": ("delta = (do * o).sum(axis=1)", "delta = (do * (p @ v)).sum(axis=1)"),
}


def mutated(name):
    old, new = MUTATIONS[name]
    assert SOURCE.count(old) >= 1, f"mutation {name} does not apply"
    mod = types.ModuleType(f"dropout_mutant_{name}")
    exec(compile(SOURCE.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_dropout_pin_catches_mutation(name):
    mod = mutated(name)
    res = {}
    for pin in ALL:
        try:
            with np.errstate(all="ignore"):
                res[pin.__name__] = bool(pin(mod))
        except Exception:
            res[pin.__name__] = False
    assert not all(res.values()), f"no pin caught {name}: {res}"
