"""CPU fp64 oracle for attention with dropout on the probabilities.

TEST INFRASTRUCTURE. Like oracle.attention, this is the checker, not the
product: only the tests, the smoke check and the bench's CPU-baseline leg may
import or call it, and it never imports anything from the HIP side.

What it computes. The page "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com),
section "Flash Attention", lists dropout with masking and softmax among the
elementwise steps whose HBM traffic the fused kernel removes. Dropout acts on
the probabilities after the softmax: with keep mask M (M_ij = 1 with
probability 1 - p) and r = 1 / (1 - p),

    O = (P * M * r) V,        LSE unchanged (taken before dropout),

and the backward pass of L = sum(O * dO) is

    dV = (P * M * r)^T dO,   dPd = dO V^T,   Delta_i = sum_d dO_id O_id,
    dS = P * (M * r * dPd - Delta),   dQ = scale dS K,   dK = scale dS^T Q

(Delta_i = sum_j P_ij M_ij r dPd_ij, since O_i = sum_j P_ij M_ij r v_j).

The mask is drawn, so that the fused backward pass can regenerate it instead
of storing it, from a counter-based generator: Philox4x32-10 (Salmon, Moraes,
Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011),
written here from that definition. One call covers a 4 x 4 block of
(query row, key) pairs:

    counter = (j // 4, i // 4, b * Hq + h, 0),  key = (seed mod 2^32, seed >> 32)
    byte 4 * (i % 4) + (j % 4) of the 128-bit output (word i % 4, byte j % 4,
    little-endian within the word) is u_ij in 0..255; keep iff u_ij >= t,
    t = round(256 p) clamped to 0..255,

so p is taken as t / 256 (probabilities are resolved in steps of 1/256) and
r = 256 / (256 - t). Rows and keys are positions in the sequence.
"""
from __future__ import annotations

import numpy as np

from oracle.attention import causal_mask, kv_head_of, softmax_rows

M0, M1 = 0xD2511F53, 0xCD9E8D57      # Philox 4x32 multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85      # Weyl key increments
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds, elementwise over uint32-valued arrays (returned as uint64 arrays).

    A round multiplies c0 and c2 by the two constants (64-bit products split
    into high and low words) and forms
        (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0));
    the key advances by the Weyl increments between rounds.
    """
    c = [np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3)]
    k0 = np.uint64(k0) & MASK32
    k1 = np.uint64(k1) & MASK32
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(W0)) & MASK32
            k1 = (k1 + np.uint64(W1)) & MASK32
        p0 = c[0] * np.uint64(M0)
        p1 = c[2] * np.uint64(M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def threshold(p):
    """Byte threshold t of a dropout probability p: p is taken as t / 256."""
    return int(min(255, max(0, round(256 * float(p)))))


def keep_mask(b, h, hq, rows, cols, p, seed):
    """Boolean keep mask [len(rows), len(cols)] of query head h of batch b."""
    t = threshold(p)
    rows = np.asarray(rows, dtype=np.uint64)
    cols = np.asarray(cols, dtype=np.uint64)
    r4 = (rows // np.uint64(4))[:, None] + np.zeros((1, len(cols)), dtype=np.uint64)
    k4 = (cols // np.uint64(4))[None, :] + np.zeros((len(rows), 1), dtype=np.uint64)
    words = philox4x32_10(k4, r4, np.uint64(b * hq + h), np.uint64(0), seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(words)                                       # [4, rows, cols]
    sel = (rows % np.uint64(4)).astype(np.int64)[:, None] + np.zeros((1, len(cols)), dtype=np.int64)
    word = np.take_along_axis(w, sel[None], axis=0)[0]
    byte = (word >> (np.uint64(8) * (cols % np.uint64(4)))[None, :]) & np.uint64(0xFF)
    return byte >= np.uint64(t)


def rescale(p):
    """1 / (1 - t / 256) for the threshold t of p."""
    return 256.0 / (256 - threshold(p))


def head_forward_backward(q, k, v, do, scale, causal, mask, r):
    """One head with a given keep mask [S, S] and rescale r: O, LSE and the gradients."""
    S = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(causal_mask(np.arange(S), S), s, -np.inf)
    p, lse = softmax_rows(s)
    pd = p * mask * r
    o = pd @ v
    dpd = do @ v.T
    delta = (do * o).sum(axis=1)
    ds = p * (mask * r * dpd - delta[:, None])
    return {"o": o, "lse": lse, "dq": scale * ds @ k, "dk_part": scale * ds.T @ q, "dv_part": pd.T @ do}


def backward(q, k, v, do, scale, causal, p, seed, masks=None):
    """Forward and backward of dropout attention over [B, H, S, D] float64 inputs.

    masks, if given, overrides the generator: a function (b, h) -> keep mask [S, S].
    """
    B, hq, S, D = q.shape
    hkv = k.shape[1]
    r = rescale(p)
    out = {"o": np.zeros_like(q), "lse": np.zeros((B, hq, S)), "dq": np.zeros_like(q),
           "dk": np.zeros_like(k), "dv": np.zeros_like(v)}
    for b in range(B):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            m = masks(b, h) if masks else keep_mask(b, h, hq, np.arange(S), np.arange(S), p, seed)
            res = head_forward_backward(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal, m, r)
            out["o"][b, h], out["lse"][b, h], out["dq"][b, h] = res["o"], res["lse"], res["dq"]
            out["dk"][b, g] += res["dk_part"]
            out["dv"][b, g] += res["dv_part"]
    return out
