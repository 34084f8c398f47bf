"""CPU fp64 oracle for attention on one (query block, key/value block) pair.

TEST INFRASTRUCTURE. Like oracle.attention, this is the checker, not the
product: only the tests, the smoke check and the bench's CPU-baseline leg may
import or call it, and it never imports anything from the HIP side.

What it computes. The page "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com),
section "Flash Attention", cuts the scores into blocks that fit on chip and
combines them with an online softmax. Sequence (context) parallel training,
which the AMD MI300X pages run at 32k and 128k tokens with context-parallel
degrees of 2 and 8 (the MoE training page, section 4.1), applies the same
cut across GPUs: each GPU holds a block of queries and sees the key/value
blocks of the sequence one at a time. The unit of that work is plain attention
between a query block and a key/value block placed at global positions:

    query row i sits at position q_pos0 + i, key j at k_pos0 + j,
    s_ij = scale * <q_i, k_j>, hidden when causal and k_pos0 + j > q_pos0 + i,
    O_b  = softmax(s) V,  LSE_b,i = ln sum_j exp(s_ij)

A row that sees no key of the block (possible once the positions are offset)
has no softmax: its partial output is 0 and its LSE is -inf, so it drops out
of the merge below.

Blocks over disjoint key sets combine exactly by their log-sum-exps:

    LSE = ln sum_b exp(LSE_b),  O = sum_b exp(LSE_b - LSE) O_b

and the backward pass of the whole row splits over the blocks the same way:
with the merged O and LSE, P_ij = exp(s_ij - LSE_i) and Delta_i = sum_d dO_id O_id
are global, and block b contributes dQ_b = scale dS K_b, dK_b = scale dS^T Q,
dV_b = P^T dO with dS = P * (dP - Delta), dP = dO V_b^T. Summing dQ_b over the
blocks gives the full dQ; dK_b, dV_b are the gradients of that block's keys
and values coming from this query block.

Everything is float64 with materialised scores; GQA heads are grouped as in
oracle.attention.
"""
from __future__ import annotations

import numpy as np

from oracle.attention import kv_head_of


def visible(n_q, n_k, causal, q_pos0, k_pos0):
    """Boolean [n_q, n_k]: key j visible to query row i (global positions)."""
    if not causal:
        return np.ones((n_q, n_k), dtype=bool)
    return (k_pos0 + np.arange(n_k))[None, :] <= (q_pos0 + np.arange(n_q))[:, None]


def head_forward_block(q, k, v, scale, causal, q_pos0, k_pos0):
    """Partial output and log-sum-exp of one head on one block pair.

    Rows that see no key get O = 0 and LSE = -inf.
    """
    vis = visible(q.shape[0], k.shape[0], causal, q_pos0, k_pos0)
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, np.where(vis, s, -np.inf).max(axis=1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    safe_l = np.where(any_vis, l, 1.0)
    o = (e / safe_l[:, None]) @ v
    lse = np.where(any_vis, m + np.log(safe_l), -np.inf)
    return o, lse


def forward_block(q, k, v, scale, causal, q_pos0, k_pos0):
    """q [B,Hq,Sq,D], k/v [B,Hkv,Sk,D] (float64) -> partial o [B,Hq,Sq,D], lse [B,Hq,Sq]."""
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    o = np.zeros((B, Hq, Sq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            o[b, h], lse[b, h] = head_forward_block(q[b, h], k[b, g], v[b, g], scale, causal, q_pos0, k_pos0)
    return o, lse


def merge(parts):
    """Combine partial (o_b, lse_b) over disjoint key blocks: exact log-sum-exp weights.

    A row whose every part has lse = -inf stays O = 0, LSE = -inf.
    """
    lses = np.stack([p[1] for p in parts])                 # [n, ...rows]
    m = lses.max(axis=0)
    fin = np.isfinite(m)
    m0 = np.where(fin, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m0[None]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(fin, m0 + np.log(np.where(fin, tot, 1.0)), -np.inf)
    coef = np.where(fin[None], w / np.where(fin, tot, 1.0)[None], 0.0)
    o = sum(coef[i][..., None] * parts[i][0] for i in range(len(parts)))
    return o, lse


def backward_block(q, k, v, o, do, lse, scale, causal, q_pos0, k_pos0):
    """Contributions of one key/value block to the gradients, given the merged o, lse.

    Returns dq_b [B,Hq,Sq,D] (to be summed over blocks) and dk_b, dv_b
    [B,Hkv,Sk,D] (summed over the query heads of each group).
    """
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    vis = visible(Sq, Sk, causal, q_pos0, k_pos0)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            l = lse[b, h]
            fin = np.isfinite(l)
            s = scale * (q[b, h] @ k[b, g].T)
            p = np.where(vis & fin[:, None], np.exp(s - np.where(fin, l, 0.0)[:, None]), 0.0)
            delta = (do[b, h] * o[b, h]).sum(axis=1)
            dp = do[b, h] @ v[b, g].T
            ds = p * (dp - delta[:, None])
            dq[b, h] = scale * ds @ k[b, g]
            dk[b, g] += scale * ds.T @ q[b, h]
            dv[b, g] += p.T @ do[b, h]
    return {"dq": dq, "dk": dk, "dv": dv}
