"""Helpers for the GPU tests: moving seeded inputs to the device and measuring errors.

The HIP path is always called through the C ABI (tiled_attention_memory_amd),
the expected values always come from the CPU oracle or from closed forms.
"""
from __future__ import annotations

import sys

import numpy as np

# Tolerances of the headline contract, bf16 outputs against the fp64 oracle:
# max |err| 2e-2 and mean |err| 2e-3 on O, dQ, dK, dV, and 1e-3 on the fp32 LSE.
# A bf16 output cannot be closer to the exact value than half a bf16 ulp of it
# (2^-9 relative; 0.0625 at |x| = 16), which exceeds 2e-2 once |x| > 5.12 -- the
# backward workloads' dV reaches |x| = 22. Both bounds are therefore applied to
# the error beyond that unavoidable output rounding: |err_i| <= 2e-2 + ulp_i / 2,
# with ulp_i the bf16 spacing at the exact value, and mean |err| <= 2e-3 + m0,
# with m0 the mean error of the exact values themselves rounded to bf16 (the
# smallest mean any bf16 output can have; about 1e-5 to 5e-4 for the usual
# shapes, more where outputs are large).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def bf16_half_ulp(x):
    """Half the spacing of bfloat16 numbers at |x| (0 at x = 0)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)                      # x = m * 2^e, m in [0.5, 1)
    h = np.ldexp(1.0, e - 9)                # bf16 keeps 8 significant bits
    return np.where(x > 0, h, 0.0)


def say(msg):
    """Name the case before each GPU step, flushed, so a failing run shows where it was."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def errs(got, want):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    return float(d.max()), float(d.mean())


def bf16_rounding_floor(want):
    """Mean |err| of the exact values themselves rounded to bf16 (nearest even): the
    smallest mean error any bf16 output can have. Outputs of large magnitude put it
    close to the mean bound, which is absolute."""
    from oracle import attention as att
    from tiled_attention_memory_amd import workloads as wl
    w = np.asarray(want, dtype=np.float64)
    r = att.bf16_bits_to_f64(wl.f32_to_bf16_bits(w.astype(np.float32)))
    return float(np.mean(np.abs(r - w)))


def assert_close(name, got, want, max_abs=MAX_ABS, mean_abs=MEAN_ABS, allowance=None):
    """The bounds above; with `allowance` (an array like want), each element may in
    addition be off by its allowance: the change that a stated rounding of the
    inputs makes to the exact value (e.g. the two readings of rotated inputs)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - want)
    allow = 0.0 if allowance is None else np.asarray(allowance, dtype=np.float64)
    excess = float(np.max(d - bf16_half_ulp(want) - allow))
    mx, mn = float(d.max()), float(d.mean())
    floor = bf16_rounding_floor(want) + (0.0 if allowance is None else float(np.mean(allow)))
    note = "" if allowance is None else f" and the input-rounding allowance (largest {float(np.max(allow)):.3e})"
    print(f"    {name}: max|err| {mx:.3e} (beyond bf16 output rounding{note} {excess:.3e}) "
          f"mean|err| {mn:.3e} (bf16 rounding of the exact values alone{note and ', plus the mean allowance'}: "
          f"{floor:.3e})", flush=True)
    assert excess <= max_abs, f"{name}: error beyond bf16 output rounding{note} {excess:.3e} > {max_abs}"
    assert mn <= mean_abs + floor, f"{name}: mean abs error {mn:.3e} > {mean_abs} + {floor:.3e}"


def assert_lse(got, want, allowance=None):
    """|err| <= 1e-3 on the fp32 LSE, beyond a per-row allowance when one is given
    (a bound on how far a stated rounding of the inputs moves the exact LSE)."""
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), "lse: non-finite values"
    d = np.abs(got - np.asarray(want, dtype=np.float64))
    mx = float(d.max())
    if allowance is None:
        print(f"    lse: max|err| {mx:.3e}", flush=True)
        assert mx <= LSE_ABS, f"lse: max abs error {mx:.3e} > {LSE_ABS}"
        return
    excess = float(np.max(d - allowance))
    print(f"    lse: max|err| {mx:.3e} (beyond the input-rounding allowance {excess:.3e}; "
          f"largest allowance {float(np.max(allowance)):.3e})", flush=True)
    assert excess <= LSE_ABS, f"lse: error beyond the allowance {excess:.3e} > {LSE_ABS}"


def run_gpu(x, causal, scale):
    """Forward and backward on the device through the C ABI; returns device tensors."""
    import torch
    import tiled_attention_memory_amd as tam
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = tam.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = tam.backward(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return {"q": q, "k": k, "v": v, "do": do, "o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
