"""The fp64 oracle over many heads or row panels at once, in threads (test infrastructure).

The work items are independent calls of the oracle's own functions
(oracle.attention.head_backward, rows_forward_backward, cols_dkdv); this
module only hands them to a thread pool and puts the results back in place.
numpy's elementwise loops and BLAS release the GIL, so threads spread the
oracle's elementwise passes over the host's cores; BLAS is held to one thread
per worker so the two kinds of threads do not oversubscribe the host.

Panels: with a causal mask, the keys after a panel's last row are hidden from
every row of the panel, so a panel's rows need only the keys up to that row
(the exact trimming the oracle itself uses for its row panels).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import time

import numpy as np
import threadpoolctl

from oracle import attention as att


def n_workers() -> int:
    """Threads for the oracle: the cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pmap(fn, items, label=""):
    """[fn(x) for x in items] on a thread pool, BLAS at one thread per worker; prints the wall time."""
    items = list(items)
    t0 = time.perf_counter()
    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(n_workers()) as ex:
            out = list(ex.map(fn, items))
    if label:
        print(f"    oracle {label}: {len(items)} items on {n_workers()} threads, "
              f"{time.perf_counter() - t0:.1f} s", flush=True)
    return out


def groups_backward(q, k, v, do, scale, causal, groups, panel_rows=None):
    """All outputs of whole GQA groups, one query head per work item.

    q, do: [B, Hq, S, D] and k, v: [B, Hkv, S, D] float64; groups: list of
    (b, kv head). Returns one dict per group with o, lse, delta, dq of its
    query heads ([g, S, ...]) and dk, dv of its key/value head ([S, D]), the
    heads' contributions summed in head order.
    """
    hq, hkv = q.shape[1], k.shape[1]
    g = hq // hkv
    items = [(b, kvh, h) for b, kvh in groups for h in range(kvh * g, (kvh + 1) * g)]
    res = pmap(lambda t: att.head_backward(q[t[0], t[2]], k[t[0], t[1]], v[t[0], t[1]], do[t[0], t[2]],
                                           scale, causal, panel_rows),
               items, label=f"{len(groups)} group(s), {len(items)} heads")
    out = []
    for n_grp, (b, kvh) in enumerate(groups):
        rs = res[n_grp * g:(n_grp + 1) * g]
        d = {n: np.stack([r[n] for r in rs]) for n in ("o", "lse", "delta", "dq")}
        d["dk"] = np.zeros_like(k[b, kvh])
        d["dv"] = np.zeros_like(v[b, kvh])
        for r in rs:
            d["dk"] += r["dk"]
            d["dv"] += r["dv"]
        out.append(d)
    return out


def all_rows(q_h, k_g, v_g, do_h, scale, panel_rows, causal=True):
    """Exact O, LSE, Delta and dQ of every row of several heads, by row panels.

    q_h, do_h: [H, S, D] (the query heads of one key/value head k_g, v_g [S, D]).
    Returns dict of [H, S] (lse, delta) and [H, S, D] (o, dq) arrays.
    """
    H, S, D = q_h.shape
    tasks = [(h, r0, min(S, r0 + panel_rows)) for h in range(H) for r0 in range(0, S, panel_rows)]

    def one(t):
        h, r0, r1 = t
        nk = r1 if causal else S
        rows = np.arange(r0, r1)
        # rows_forward_backward indexes q and dO by absolute row number
        return att.rows_forward_backward(q_h[h], k_g[:nk], v_g[:nk], do_h[h], rows, scale, causal)

    res = pmap(one, tasks, label=f"rows of {H} heads x {S}")
    out = {"o": np.empty((H, S, D)), "dq": np.empty((H, S, D)),
           "lse": np.empty((H, S)), "delta": np.empty((H, S))}
    for (h, r0, r1), r in zip(tasks, res):
        for n in out:
            out[n][h, r0:r1] = r[n]
    return out


def key_blocks_dkdv(q_h, do_h, k_g, v_g, lse, delta, blocks, block_keys, scale, causal=True):
    """Exact dK, dV of whole key blocks [j * block_keys, (j+1) * block_keys) of one key/value head.

    lse, delta: [H, S] for every row of the H query heads (from all_rows).
    Returns {j: (dk, dv)}.
    """
    S = k_g.shape[0]

    def one(j):
        cols = np.arange(j * block_keys, min(S, (j + 1) * block_keys))
        row_lo = int(cols[0]) if causal else 0
        return att.cols_dkdv(q_h[:, row_lo:], do_h[:, row_lo:], k_g, v_g, cols, lse[:, row_lo:],
                             delta[:, row_lo:], row_lo, scale, causal)

    res = pmap(one, blocks, label=f"{len(blocks)} key blocks")
    return dict(zip(blocks, res))
