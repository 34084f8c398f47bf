"""Pins that tie the CPU oracle to something other than itself.

Each pin takes the oracle module as an argument, so the same checks run on
the real oracle (tests/test_oracle.py) and on copies of it with a planted
mistake (tests/test_oracle_mutations.py), where at least one must fail.

What each pin rests on:
  * closed forms of the softmax definition: a zero query (or zero scale)
    gives equal weights over the visible keys, i.e. the running mean of V and
    LSE_i = ln(i + 1); row 0 of a causal head sees only key 0; S = 1;
  * a worked example derived by hand from the definition (S = 3, D = 2), and a
    non-causal one (S = 2);
  * invariances of the definition: a constant added to every key leaves O
    unchanged (so the key gradients sum to zero), a constant added to every
    value is added to every output (so the value gradients sum to the
    summed output gradients);
  * central finite differences of L = sum(O * dO) in float64;
  * an independent library routine: PyTorch's CPU float64
    scaled_dot_product_attention with autograd, GQA enabled.
"""
from __future__ import annotations

import math

import numpy as np


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def close(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return a.shape == b.shape and bool(np.all(np.isfinite(a))) and float(np.max(np.abs(a - b))) <= tol


# ---------------------------------------------------------------------------
def pin_zero_query_running_mean(att):
    """Q = 0 (and scale = 0 with random Q): O_i = mean(V_0..V_i), LSE_i = ln(i+1), per GQA group."""
    B, hq, hkv, S, D = 2, 4, 2, 9, 3
    v = rand((B, hkv, S, D), 1)
    k = rand((B, hkv, S, D), 2)
    ok = True
    for q, scale in ((np.zeros((B, hq, S, D)), 0.7), (rand((B, hq, S, D), 3), 0.0)):
        o, lse = att.forward(q, k, v, scale, causal=True)
        counts = np.arange(1, S + 1)[:, None]
        for b in range(B):
            for h in range(hq):
                g = h // (hq // hkv)
                mean = np.cumsum(v[b, g], axis=0) / counts
                ok &= close(o[b, h], mean, 1e-12)
                ok &= close(lse[b, h], np.log(np.arange(1, S + 1)), 1e-12)
        # non-causal: every row is the mean of all values and LSE = ln S
        o, lse = att.forward(q, k, v, scale, causal=False)
        for b in range(B):
            for h in range(hq):
                g = h // (hq // hkv)
                ok &= close(o[b, h], np.broadcast_to(v[b, g].mean(axis=0), (S, D)), 1e-12)
                ok &= close(lse[b, h], np.full(S, math.log(S)), 1e-12)
    return ok


def pin_first_row_and_single_key(att):
    """Causal row 0 sees only key 0; with S = 1 the softmax is trivially 1."""
    B, hq, hkv, S, D = 1, 6, 3, 7, 5
    q, k, v = rand((B, hq, S, D), 4), rand((B, hkv, S, D), 5), rand((B, hkv, S, D), 6)
    scale = 0.37
    o, lse = att.forward(q, k, v, scale, causal=True)
    ok = True
    for h in range(hq):
        g = h // 2
        ok &= close(o[0, h, 0], v[0, g, 0], 1e-12)
        ok &= close(lse[0, h, 0], scale * float(q[0, h, 0] @ k[0, g, 0]), 1e-12)
    # S = 1
    q1, k1, v1, do1 = q[:, :, :1], k[:, :, :1], v[:, :, :1], rand((B, hq, 1, D), 7)
    for causal in (True, False):
        r = att.backward(q1, k1, v1, do1, scale, causal=causal)
        ok &= close(r["o"], np.repeat(v1, 2, axis=1), 1e-12)
        ok &= close(r["dq"], np.zeros_like(q1), 1e-12)
        ok &= close(r["dk"], np.zeros_like(k1), 1e-12)
        dv = do1.reshape(B, hkv, 2, 1, D).sum(axis=2)
        ok &= close(r["dv"], dv, 1e-12)
    return ok


def hand_example():
    """A causal S = 3, D = 2 head worked out by hand from the definition (scale 1).

    k0 = (0,0), k1 = (1,0), k2 = (0,1); q1 = (ln 3, 0), q2 = (ln 2, ln 5).
    Row 1 scores (0, ln 3) -> P = (1/4, 3/4), LSE = ln 4.
    Row 2 scores (0, ln 2, ln 5) -> weights (1, 2, 5)/8, LSE = ln 8.
    v = (1,0), (0,1), (2,2); dO = (1,0), (0,1), (1,1).
    dP rows: (1), (0, 1), (1, 1, 4); Delta = (1, 3/4, 23/8);
    dS rows: (0), (-3/16, 3/16), (-15/64, -15/32, 45/64).
    """
    l2, l3, l5 = math.log(2), math.log(3), math.log(5)
    q = np.array([[0.5, -0.5], [l3, 0.0], [l2, l5]])
    k = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 2.0]])
    do = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    ds = np.array([[0.0, 0.0, 0.0], [-3 / 16, 3 / 16, 0.0], [-15 / 64, -15 / 32, 45 / 64]])
    expect = {
        "o": np.array([[1.0, 0.0], [0.25, 0.75], [1.375, 1.5]]),
        "lse": np.array([0.0, math.log(4), math.log(8)]),
        "delta": np.array([1.0, 0.75, 23 / 8]),
        "dv": np.array([[1.125, 0.375], [0.25, 1.0], [0.625, 0.625]]),
        "dq": np.array([[0.0, 0.0], [3 / 16, 0.0], [-15 / 32, 45 / 64]]),
        "dk": np.array([-3 / 16 * q[1] - 15 / 64 * q[2],
                        3 / 16 * q[1] - 15 / 32 * q[2],
                        45 / 64 * q[2]]),
    }
    # row 0's LSE is q0 . k0 = 0
    return q, k, v, do, ds, expect


def pin_hand_example(att):
    q, k, v, do, _, expect = hand_example()
    r = att.backward(q[None, None], k[None, None], v[None, None], do[None, None], 1.0, causal=True)
    ok = True
    for name, val in expect.items():
        ok &= close(r[name][0, 0], val, 1e-12)
    # non-causal S = 2: q0 = (ln 3, 0) sees (0, ln 3) -> (1/4, 3/4); q1 = 0 -> (1/2, 1/2)
    q2 = np.array([[math.log(3), 0.0], [0.0, 0.0]])
    k2 = np.array([[0.0, 0.0], [1.0, 0.0]])
    v2 = np.array([[4.0, 0.0], [0.0, 8.0]])
    o, lse = att.forward(q2[None, None], k2[None, None], v2[None, None], 1.0, causal=False)
    ok &= close(o[0, 0], np.array([[1.0, 6.0], [2.0, 4.0]]), 1e-12)
    ok &= close(lse[0, 0], np.array([math.log(4), math.log(2)]), 1e-12)
    return ok


def pin_shift_invariance(att):
    """K + c leaves O unchanged and sum_j dK_j = 0; V + c shifts O by c and sum_j dV_j = sum dO."""
    B, hq, hkv, S, D = 1, 4, 2, 11, 4
    q, k, v, do = (rand((B, hq, S, D), 8), rand((B, hkv, S, D), 9), rand((B, hkv, S, D), 10),
                   rand((B, hq, S, D), 11))
    c = rand((D,), 12)
    ok = True
    for causal in (True, False):
        r = att.backward(q, k, v, do, 0.6, causal=causal)
        o_k, _ = att.forward(q, k + c, v, 0.6, causal=causal)
        o_v, _ = att.forward(q, k, v + c, 0.6, causal=causal)
        ok &= close(o_k, r["o"], 1e-12)
        ok &= close(o_v, r["o"] + c, 1e-12)
        ok &= close(r["dk"].sum(axis=2), np.zeros((B, hkv, D)), 1e-10)
        dsum = do.reshape(B, hkv, hq // hkv, S, D).sum(axis=(2, 3))
        ok &= close(r["dv"].sum(axis=2), dsum, 1e-10)
    return ok


def pin_finite_differences(att, eps=1e-6):
    """Central differences of L = sum(O * dO) against the analytic gradients."""
    B, hq, hkv, S, D = 1, 4, 2, 5, 3
    q, k, v, do = (rand((B, hq, S, D), 13), rand((B, hkv, S, D), 14), rand((B, hkv, S, D), 15),
                   rand((B, hq, S, D), 16))
    scale = 0.8
    ok = True
    for causal in (True, False):
        r = att.backward(q, k, v, do, scale, causal=causal)

        def loss(qq, kk, vv):
            return float(np.sum(att.forward(qq, kk, vv, scale, causal=causal)[0] * do))

        for name, x in (("dq", q), ("dk", k), ("dv", v)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
                args_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            ok &= close(r[name], num, 1e-7 * max(1.0, float(np.max(np.abs(num)))))
    return ok


def torch_reference(q, k, v, do, scale, causal):
    """PyTorch CPU float64 SDPA (GQA enabled) and autograd gradients, plus its logsumexp."""
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    o.backward(torch.tensor(do, dtype=torch.float64))
    g = q.shape[1] // k.shape[1]
    with torch.no_grad():
        kr = tk.repeat_interleave(g, dim=1)
        s = scale * torch.matmul(tq, kr.transpose(-1, -2))
        if causal:
            S = q.shape[2]
            s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
        lse = torch.logsumexp(s, dim=-1)
    return {"o": o.detach().numpy(), "lse": lse.numpy(), "dq": tq.grad.numpy(),
            "dk": tk.grad.numpy(), "dv": tv.grad.numpy()}


def pin_torch_sdpa(att, shapes=((1, 4, 2, 6, 3), (2, 6, 3, 17, 8), (1, 8, 1, 33, 16))):
    ok = True
    for i, (B, hq, hkv, S, D) in enumerate(shapes):
        q, k, v, do = (rand((B, hq, S, D), 20 + i), rand((B, hkv, S, D), 30 + i),
                       rand((B, hkv, S, D), 40 + i), rand((B, hq, S, D), 50 + i))
        scale = 1.0 / math.sqrt(D)
        for causal in (True, False):
            r = att.backward(q, k, v, do, scale, causal=causal)
            t = torch_reference(q, k, v, do, scale, causal)
            for name in ("o", "lse", "dq", "dk", "dv"):
                ok &= close(r[name], t[name], 1e-10)
    return ok


ALL_PINS = [pin_zero_query_running_mean, pin_first_row_and_single_key, pin_hand_example,
            pin_shift_invariance, pin_finite_differences, pin_torch_sdpa]
