"""CPU fp64 oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE. This module is the checker, not the product. Only the
tests, the smoke check and the bench's CPU-baseline leg may import or call it;
the HIP library never does, and it never imports anything from the HIP side.

What it computes. The page "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com),
section "Flash Attention", describes the method: standard attention is bound by
HBM traffic of its elementwise steps (masking, softmax, dropout), and Flash
Attention fixes that with kernel fusion, tiling with an online softmax, and
recomputation in the backward pass. Those three techniques change where the
intermediate values live, not the result, so this oracle computes the plain
definition they all reproduce and uses none of them:

    s_ij = scale * <q_i, k_j>,  masked to -inf where j > i when causal
    P    = row-wise softmax(s),  LSE_i = ln sum_j exp(s_ij)
    O    = P V

with grouped-query heads: query head h reads key/value head h // (Hq / Hkv).
The backward pass differentiates L = sum(O * dO):

    dV = P^T dO,  dP = dO V^T,  Delta_i = sum_j P_ij dP_ij,
    dS = P * (dP - Delta),  dQ = scale * dS K,  dK = scale * dS^T Q

with dK and dV summed over the query heads that share a key/value head.

Everything is float64 and the full score matrix of a head is materialised
(optionally in whole-row panels for very long sequences, see head_forward).
The page prints no dropout probability for this path and none is applied.

Readings where the page is silent (GQA grouping, mask alignment, LSE base,
layout) are: contiguous head groups, key j visible to query i iff j <= i,
natural-log LSE, [B, H, S, D] row-major.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# input decoding
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: the pattern is the top half of a float32."""
    u = np.ascontiguousarray(bits).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """Key/value head read by query head h (contiguous groups of hq // hkv heads)."""
    return h // (hq // hkv)


# ----------------------------------------------------------------------------
# one head, materialised scores ("Flash Attention" section: the N x N scores)
# ----------------------------------------------------------------------------
def causal_mask(rows: np.ndarray, n_keys: int) -> np.ndarray:
    """Boolean [len(rows), n_keys]: True where key j is visible to query row i (j <= i)."""
    return np.arange(n_keys)[None, :] <= rows[:, None]


def masked_scores(q_rows, k, scale, causal, rows):
    """s = scale * q k^T for the given query rows, -inf where the causal mask hides a key."""
    s = scale * (q_rows @ k.T)
    if causal:
        s = np.where(causal_mask(rows, k.shape[0]), s, -np.inf)
    return s


def softmax_rows(s):
    """Row softmax of masked scores and the row log-sum-exp (natural log).

    Uses the usual max subtraction; a row whose keys are all masked is not
    produced by square causal attention and is not handled.
    """
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def _panels(S, causal, panel_rows):
    """Whole-row panels [r0, r1) and the number of keys each needs.

    With a causal mask, keys past the panel's last row are masked for every row
    of the panel: leaving them out drops terms that are exactly zero.
    """
    step = S if panel_rows is None else panel_rows
    for r0 in range(0, S, step):
        r1 = min(S, r0 + step)
        yield r0, r1, (r1 if causal else S)


def head_forward(q, k, v, scale, causal, panel_rows=None):
    """O [S, D] and LSE [S] of one query head against its key/value head."""
    S = q.shape[0]
    o = np.empty_like(q)
    lse = np.empty(S)
    for r0, r1, nk in _panels(S, causal, panel_rows):
        rows = np.arange(r0, r1)
        p, lse[r0:r1] = softmax_rows(masked_scores(q[r0:r1], k[:nk], scale, causal, rows))
        o[r0:r1] = p @ v[:nk]
    return o, lse


def head_backward(q, k, v, do, scale, causal, panel_rows=None):
    """Gradients of L = sum(O * dO) for one query head (recomputes P from scratch).

    Returns dict(o, lse, delta, dq, dk, dv); dk and dv are this head's
    contribution to its key/value head.
    """
    S = q.shape[0]
    out = {"o": np.empty_like(q), "lse": np.empty(S), "delta": np.empty(S),
           "dq": np.empty_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v)}
    for r0, r1, nk in _panels(S, causal, panel_rows):
        rows = np.arange(r0, r1)
        kk, vv = k[:nk], v[:nk]
        p, out["lse"][r0:r1] = softmax_rows(masked_scores(q[r0:r1], kk, scale, causal, rows))
        out["o"][r0:r1] = p @ vv
        dpo = do[r0:r1]
        out["dv"][:nk] += p.T @ dpo
        dp = dpo @ vv.T
        delta = (p * dp).sum(axis=1)
        out["delta"][r0:r1] = delta
        ds = p * (dp - delta[:, None])
        out["dq"][r0:r1] = scale * (ds @ kk)
        out["dk"][:nk] += scale * (ds.T @ q[r0:r1])
    return out


# ----------------------------------------------------------------------------
# whole tensors [B, H, S, D]
# ----------------------------------------------------------------------------
def forward(q, k, v, scale, causal=True, panel_rows=None):
    """O [B,Hq,S,D] and LSE [B,Hq,S] (float64) for float64 inputs."""
    B, hq, S, D = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    o = np.empty_like(q)
    lse = np.empty((B, hq, S))
    for b in range(B):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            o[b, h], lse[b, h] = head_forward(q[b, h], k[b, g], v[b, g], scale, causal, panel_rows)
    return o, lse


def backward(q, k, v, do, scale, causal=True, panel_rows=None, heads=None):
    """Forward outputs and all gradients (float64).

    heads: optional list of (b, kv_head) groups to compute; dq/o/lse/delta are
    then filled only for those groups' query heads (NaN elsewhere), and dk/dv
    only for those groups (NaN elsewhere).
    """
    B, hq, S, D = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    g_size = hq // hkv
    full = heads is None
    groups = [(b, g) for b in range(B) for g in range(hkv)] if full else list(heads)
    fill = 0.0 if full else np.nan
    res = {"o": np.full_like(q, fill), "lse": np.full((B, hq, S), fill),
           "delta": np.full((B, hq, S), fill), "dq": np.full_like(q, fill),
           "dk": np.full_like(k, fill), "dv": np.full_like(v, fill)}
    for b, g in groups:
        res["dk"][b, g] = 0.0
        res["dv"][b, g] = 0.0
        for h in range(g * g_size, (g + 1) * g_size):
            assert kv_head_of(h, hq, hkv) == g
            r = head_backward(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal, panel_rows)
            for name in ("o", "lse", "delta", "dq"):
                res[name][b, h] = r[name]
            res["dk"][b, g] += r["dk"]
            res["dv"][b, g] += r["dv"]
    return res


# ----------------------------------------------------------------------------
# sampled evaluation for sequences too long to materialise in a test
# ----------------------------------------------------------------------------
def rows_forward_backward(q_h, k_g, v_g, do_h, rows, scale, causal=True):
    """Exact O, LSE, Delta and dQ of selected query rows of one head.

    A row's outputs and its dQ depend only on its own score row, so each row is
    the definition applied to that row alone.
    """
    rows = np.asarray(rows)
    s = masked_scores(q_h[rows], k_g, scale, causal, rows)
    p, lse = softmax_rows(s)
    dp = do_h[rows] @ v_g.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    return {"o": p @ v_g, "lse": lse, "delta": delta, "dq": scale * (ds @ k_g)}


def cols_dkdv(q_heads, do_heads, k_g, v_g, cols, lse_heads, delta_heads, row_lo, scale,
              causal=True):
    """Exact dK, dV of selected key rows of one key/value head.

    q_heads, do_heads: [g, R, D] query rows row_lo..row_lo+R-1 of each query head
    in the group; lse_heads, delta_heads: [g, R] for those rows (from
    rows_forward_backward). Every query row that can see a selected key must
    be inside [row_lo, row_lo + R): with a causal mask that means row_lo <= min(cols);
    without one, all S rows.
    """
    cols = np.asarray(cols)
    R = q_heads.shape[1]
    rows = np.arange(row_lo, row_lo + R)
    if causal:
        assert row_lo <= cols.min()
    else:
        assert row_lo == 0 and R == k_g.shape[0]
    dk = np.zeros((len(cols), k_g.shape[1]))
    dv = np.zeros((len(cols), v_g.shape[1]))
    for h in range(q_heads.shape[0]):
        s = scale * (q_heads[h] @ k_g[cols].T)              # [R, C]
        if causal:
            s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
        p = np.exp(s - lse_heads[h][:, None])
        dp = do_heads[h] @ v_g[cols].T
        ds = p * (dp - delta_heads[h][:, None])
        dv += p.T @ do_heads[h]
        dk += scale * (ds.T @ q_heads[h])
    return dk, dv
