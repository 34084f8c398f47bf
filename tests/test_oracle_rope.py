"""CPU checks of the RoPE oracle (oracle.rope): closed forms of the rotation, the
relative-position property that motivates it, gradients against torch, and planted
mistakes that these checks must catch."""
import inspect
import types

import numpy as np
import pytest

from oracle import rope
from oracle_pins import close, rand


def pin_closed_forms(mod):
    """Position 0 is the identity; D = 2 is a plane rotation by m radians; the inverse undoes it."""
    x = rand((1, 2, 5, 8), 91)
    ok = close(mod.rotate(x[:, :, :1], [0], 10000.0), x[:, :, :1], 0)
    v = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]])          # two heads, one row, D = 2
    m = 0.7
    want = np.array([[[[np.cos(m), np.sin(m)]], [[-np.sin(m), np.cos(m)]]]])
    ok &= close(mod.rotate(v, [m], 10000.0), want, 1e-15)
    ok &= close(mod.rotate(mod.rotate(x, np.arange(5) + 3, 1e6), np.arange(5) + 3, 1e6, inverse=True), x, 1e-12)
    # frequencies: dimension pair d turns by m * base^(-2d/D)
    a = mod.angles([10], 8, 100.0)
    ok &= close(a, [[10.0, 10.0 / 100 ** 0.25, 10.0 / 100 ** 0.5, 10.0 / 100 ** 0.75]], 1e-12)
    # norms are kept
    ok &= close(np.linalg.norm(mod.rotate(x, np.arange(5), 1e4), axis=-1), np.linalg.norm(x, axis=-1), 1e-12)
    return ok


def pin_relative_positions(mod):
    """<R_m q, R_n k> depends only on m - n (the reason for the rotation)."""
    q, k = rand((1, 1, 1, 16), 92), rand((1, 1, 1, 16), 93)
    dots = []
    for m, n in ((5, 2), (105, 102), (1003, 1000)):
        dots.append(float((mod.rotate(q, [m], 1e4) * mod.rotate(k, [n], 1e4)).sum()))
    return max(dots) - min(dots) <= 1e-10


def pin_gradients_against_torch(mod):
    import torch
    B, hq, hkv, S, D = 1, 4, 2, 11, 8
    q, k, v, do = rand((B, hq, S, D), 94), rand((B, hkv, S, D), 95), rand((B, hkv, S, D), 96), rand((B, hq, S, D), 97)
    base = 1e4
    r = mod.backward(q, k, v, do, 0.4, True, base, bf16_rotated=False)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    pos = torch.arange(S, dtype=torch.float64)
    inv = base ** (-2.0 * torch.arange(D // 2, dtype=torch.float64) / D)
    a = pos[:, None] * inv[None, :]
    c, s = torch.cos(a), torch.sin(a)

    def rot(x):
        lo, hi = x[..., : D // 2], x[..., D // 2:]
        return torch.cat([lo * c - hi * s, hi * c + lo * s], dim=-1)

    o = torch.nn.functional.scaled_dot_product_attention(rot(tq), rot(tk), tv, is_causal=True, scale=0.4,
                                                         enable_gqa=True)
    o.backward(torch.tensor(do))
    return (close(r["o"], o.detach().numpy(), 1e-12) and close(r["dq"], tq.grad.numpy(), 1e-11)
            and close(r["dk"], tk.grad.numpy(), 1e-11) and close(r["dv"], tv.grad.numpy(), 1e-11))


def pin_round_bf16(mod):
    """Ties go to the even neighbour, other values to the nearest one (spacing 2^-7 on [1, 2));
    agrees with rounding the float32 bit pattern on values that are exact in float32."""
    r = mod.round_bf16
    ok = r(1 + 2.0 ** -8) == 1.0 and r(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    ok &= r(1 + 2.0 ** -8 + 2.0 ** -20) == 1 + 2.0 ** -7 and r(-(1 + 3 * 2.0 ** -8)) == -(1 + 2.0 ** -6)
    ok &= r(0.0) == 0.0 and r(3.0) == 3.0 and r(2.0 ** -130) == 2.0 ** -130
    x = rand((4096,), 98).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    ok &= bool(np.array_equal(r(x.astype(np.float64)), bits.astype(np.uint32).view(np.float32).astype(np.float64)))
    return ok


ALL = [pin_closed_forms, pin_relative_positions, pin_gradients_against_torch, pin_round_bf16]


@pytest.mark.parametrize("pin", ALL, ids=lambda p: p.__name__)
def test_rope_pin(pin):
    assert pin(rope)


SOURCE = inspect.getsource(rope)
MUTATIONS = {
    "interleaved_pairs": ("lo, hi = x[..., : D // 2], x[..., D // 2:]", "lo, hi = x[..., 0::2], x[..., 1::2]"),
    "sign_of_sine": ("[lo * c - hi * s, hi * c + lo * s]", "[lo * c + hi * s, hi * c - lo * s]"),
    "frequency_exponent": ("-2.0 * d / D", "-d / D"),
    "gradient_not_rotated_back": ('"dq": rotate(r["dq"], pos, base, inverse=True)', '"dq": r["dq"]'),
    "round_ties_up": ("np.rint(m * 256.0)", "np.floor(m * 256.0 + 0.5)"),
    "key_positions_reversed": ("qr, kr = rotate(q, pos, base), rotate(k, pos, base)",
                               "qr, kr = rotate(q, pos, base), rotate(k, pos[::-1], base)"),
}


def mutated(name):
    old, new = MUTATIONS[name]
    assert SOURCE.count(old) >= 1, f"mutation {name} does not apply"
    mod = types.ModuleType(f"rope_mutant_{name}")
    exec(compile(SOURCE.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_rope_pin_catches_mutation(name):
    mod = mutated(name)
    res = {}
    for pin in ALL:
        try:
            with np.errstate(all="ignore"):
                res[pin.__name__] = bool(pin(mod))
        except Exception:
            res[pin.__name__] = False
    assert not all(res.values()), f"no pin caught {name}: {res}"
