"""CPU fp64 oracle for attention with rotary position embedding (RoPE) on Q and K.

TEST INFRASTRUCTURE. Like oracle.attention, this is the checker, not the
product: only the tests, the smoke check and the bench's CPU-baseline leg may
import or call it, and it never imports anything from the HIP side.

What it computes. The AMD MI300X MoE training page trains with rotary
embeddings of base theta = 10^6 (its model configuration); the rotation is
applied to Q and K just before the product Q K^T that the page "使用 PyTorch
FSDP 微調 Llama 2 70B" (agentlenshq.com), section "Flash Attention", fuses.
With position m of a row and the rotate-half pairing (dimension d with
d + D/2, the convention of the Llama and GPT-NeoX implementations):

    a_d = m * base^(-2d/D),   d = 0 .. D/2 - 1
    x'_d       = x_d cos a_d - x_{d+D/2} sin a_d
    x'_{d+D/2} = x_{d+D/2} cos a_d + x_d sin a_d

Attention then runs on (Q', K', V). Since the rotation R_m is orthogonal and
linear, the gradients with respect to the unrotated inputs are R_m^T applied
to the gradients with respect to Q' and K' (the inverse rotation).
Row i of the sequence sits at position i. (A common offset of all positions
would change nothing: the scores depend on position differences only.)

Precision. The attention inputs are bf16 tensors, and so are the rotated Q
and K that feed the products when the rotation runs ahead of them (as its own
step on bf16 tensors, or fused into the load of the attention kernel): by
default the rotated values are rounded to bf16, nearest with ties to even,
and the gradient treats that rounding as the identity.
"""
from __future__ import annotations

import numpy as np

from oracle import attention as att


def angles(positions, D, base):
    """a[m, d] = positions[m] * base^(-2d/D) for d < D/2 (float64)."""
    d = np.arange(D // 2, dtype=np.float64)
    return np.asarray(positions, dtype=np.float64)[:, None] * np.power(float(base), -2.0 * d / D)[None, :]


def rotate(x, positions, base, inverse=False):
    """Rotate the last axis of x [..., S, D] by the angles of the S positions (or the inverse rotation)."""
    D = x.shape[-1]
    a = angles(positions, D, base)
    c, s = np.cos(a), np.sin(a)
    if inverse:
        s = -s
    lo, hi = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def round_bf16(x):
    """Nearest bfloat16 value (8 significant bits, ties to even) of float64 values."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                    # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def backward(q, k, v, do, scale, causal, base, bf16_rotated=True):
    """Forward and backward of attention on RoPE-rotated Q and K ([B, H, S, D] float64).

    Returns o, lse and the gradients with respect to the unrotated q, k and v.
    """
    S = q.shape[2]
    pos = np.arange(S)
    qr, kr = rotate(q, pos, base), rotate(k, pos, base)
    if bf16_rotated:
        qr, kr = round_bf16(qr), round_bf16(kr)
    r = att.backward(qr, kr, v, do, scale, causal=causal)
    return {"o": r["o"], "lse": r["lse"], "dq": rotate(r["dq"], pos, base, inverse=True),
            "dk": rotate(r["dk"], pos, base, inverse=True), "dv": r["dv"], "q_rot": qr, "k_rot": kr}
