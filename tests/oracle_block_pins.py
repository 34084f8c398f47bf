"""Pins for the block oracle (oracle.blocks), each a function of the module under test.

The block oracle is checked against things it does not compute itself:
- the square-sequence oracle (oracle.attention, pinned on its own by
  oracle_pins.py): cutting one sequence into query and key blocks at their
  global positions, merging the partial results and summing the partial
  gradients must give back the whole-sequence result;
- PyTorch's CPU float64 scaled_dot_product_attention with an explicit boolean
  mask for offset, rectangular blocks, with autograd for the gradients;
- the closed form of a block whose keys all lie after its queries.
Each returns True when the pin holds.
"""
import math

import numpy as np

from oracle import attention as att
from oracle_pins import close, rand


def _split(n, cuts):
    edges = [0, *cuts, n]
    return [(edges[i], edges[i + 1]) for i in range(len(edges) - 1)]


def pin_partition_forward(blk):
    """Merged key blocks give the square oracle's rows of the query block, causal or not."""
    ok = True
    B, hq, hkv, S, D = 1, 4, 2, 37, 8
    q, k, v = rand((B, hq, S, D), 1), rand((B, hkv, S, D), 2), rand((B, hkv, S, D), 3)
    scale = 1.0 / math.sqrt(D)
    for causal in (True, False):
        full_o, full_lse = att.forward(q, k, v, scale, causal=causal)
        for q0, q1 in _split(S, [10, 29]):
            parts = [blk.forward_block(q[:, :, q0:q1], k[:, :, k0:k1], v[:, :, k0:k1], scale, causal, q0, k0)
                     for k0, k1 in _split(S, [7, 20])]
            o, lse = blk.merge(parts)
            ok &= close(o, full_o[:, :, q0:q1], 1e-12) and close(lse, full_lse[:, :, q0:q1], 1e-12)
    return ok


def pin_partition_backward(blk):
    """Partial gradients summed over blocks give the square oracle's dQ, dK, dV."""
    ok = True
    B, hq, hkv, S, D = 1, 4, 2, 29, 8
    q, k, v, do = (rand((B, hq, S, D), 11), rand((B, hkv, S, D), 12), rand((B, hkv, S, D), 13),
                   rand((B, hq, S, D), 14))
    scale = 0.4
    for causal in (True, False):
        full = att.backward(q, k, v, do, scale, causal=causal)
        qb, kb = _split(S, [13]), _split(S, [5, 18])
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for q0, q1 in qb:
            o, lse = full["o"][:, :, q0:q1], full["lse"][:, :, q0:q1]
            for k0, k1 in kb:
                g = blk.backward_block(q[:, :, q0:q1], k[:, :, k0:k1], v[:, :, k0:k1], o, do[:, :, q0:q1], lse,
                                       scale, causal, q0, k0)
                dq[:, :, q0:q1] += g["dq"]
                dk[:, :, k0:k1] += g["dk"]
                dv[:, :, k0:k1] += g["dv"]
        ok &= close(dq, full["dq"], 1e-11) and close(dk, full["dk"], 1e-11) and close(dv, full["dv"], 1e-11)
    return ok


def pin_torch_masked_block(blk):
    """An offset rectangular block against torch SDPA with an explicit mask (one block = whole row)."""
    import torch
    ok = True
    B, hq, hkv, Sq, Sk, D = 1, 4, 2, 9, 13, 8
    q0, k0 = 20, 15            # rows 20..28 see keys 15..min(row, 27)
    q, k, v, do = (rand((B, hq, Sq, D), 21), rand((B, hkv, Sk, D), 22), rand((B, hkv, Sk, D), 23),
                   rand((B, hq, Sq, D), 24))
    scale = 0.3
    mask = (k0 + np.arange(Sk))[None, :] <= (q0 + np.arange(Sq))[:, None]
    assert mask.any(axis=1).all()
    o, lse = blk.forward_block(q, k, v, scale, True, q0, k0)
    g = blk.backward_block(q, k, v, o, do, lse, scale, True, q0, k0)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(mask), scale=scale,
                                                          enable_gqa=True)
    to.backward(torch.tensor(do))
    with torch.no_grad():
        s = scale * torch.matmul(tq, tk.repeat_interleave(hq // hkv, dim=1).transpose(-1, -2))
        tl = torch.logsumexp(s.masked_fill(~torch.tensor(mask), float("-inf")), dim=-1)
    ok &= close(o, to.detach().numpy(), 1e-12) and close(lse, tl.numpy(), 1e-12)
    ok &= close(g["dq"], tq.grad.numpy(), 1e-11) and close(g["dk"], tk.grad.numpy(), 1e-11)
    ok &= close(g["dv"], tv.grad.numpy(), 1e-11)
    return ok


def pin_fully_hidden_block(blk):
    """Keys all after the queries: O = 0, LSE = -inf, zero gradients, and the merge ignores it."""
    B, hq, hkv, Sq, Sk, D = 1, 2, 1, 4, 6, 8
    q, k, v, do = (rand((B, hq, Sq, D), 31), rand((B, hkv, Sk, D), 32), rand((B, hkv, Sk, D), 33),
                   rand((B, hq, Sq, D), 34))
    o, lse = blk.forward_block(q, k, v, 0.5, True, 3, 10)
    ok = bool(np.all(o == 0.0)) and bool(np.all(np.isneginf(lse)))
    k2, v2 = rand((B, hkv, 3, D), 35), rand((B, hkv, 3, D), 36)
    other = blk.forward_block(q, k2, v2, 0.5, True, 3, 0)
    mo, ml = blk.merge([(o, lse), other])
    ok &= close(mo, other[0], 1e-15) and close(ml, other[1], 1e-15)
    g = blk.backward_block(q, k, v, mo, do, ml, 0.5, True, 3, 10)
    ok &= all(bool(np.all(g[n] == 0.0)) for n in ("dq", "dk", "dv"))
    return ok


ALL_BLOCK_PINS = [pin_partition_forward, pin_partition_backward, pin_torch_masked_block, pin_fully_hidden_block]
