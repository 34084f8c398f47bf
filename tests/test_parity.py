"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (bf16 outputs vs fp64): max |err| <= 2e-2 and mean |err| <= 2e-3 on
O, dQ, dK, dV, each beyond the rounding a bf16 output cannot avoid (see
gpu_helpers.assert_close); |err| <= 1e-3 on the fp32 LSE.

Small shapes are compared element by element in full; they span several tiles
and ragged tails (S not a multiple of the 64/128-row tiles), GQA group sizes
1..16, both head dims, causal and not. The five named workloads run at their
full sizes in the same launch configuration the bench times:
  * S = 256 and the batch-16 S = 64 workload: every element;
  * S = 4096 (64/8 heads): every element of all eight GQA groups;
  * S = 32768 (K x 3): one whole GQA group element by element (every row of
    O, LSE, dQ of its four query heads, every key row of dK, dV);
  * S = 81920 (8/1 heads): every row of O, LSE and dQ, and dK, dV on eight
    whole 128-key blocks (first, last, six seeded), which the oracle computes
    exactly from every row's LSE and Delta;
plus, for the two long ones, the shift-invariance sums over every key row.
The oracle runs in threads over heads and row panels (oracle_par).
"""
import math

import numpy as np
import pytest

import oracle_par as par
from gpu_helpers import assert_close, assert_lse, run_gpu, say, to_f64
from oracle import attention as att
from tiled_attention_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu

SMALL = [  # B, Hq, Hkv, S, D, causal
    (1, 1, 1, 1, 64, True), (1, 1, 1, 2, 128, True), (1, 2, 1, 63, 64, True),
    (1, 4, 2, 64, 128, True), (2, 4, 2, 65, 128, True), (1, 8, 1, 127, 128, True),
    (1, 6, 3, 129, 64, True), (1, 4, 4, 200, 128, True), (1, 16, 4, 333, 128, True),
    (2, 2, 2, 256, 64, True), (1, 4, 1, 640, 128, True), (1, 2, 2, 1000, 64, True),
    (1, 1, 1, 1, 128, False), (1, 8, 8, 100, 128, False), (1, 4, 2, 257, 64, False),
    (2, 6, 2, 190, 128, False), (1, 2, 1, 520, 128, False),
    # up to 64 (32) rows, 2 (4) query heads of a group share a unit of the
    # query-stationary kernels; an odd group keeps one head per unit
    (2, 8, 2, 20, 128, True), (1, 8, 1, 32, 64, False), (3, 4, 1, 33, 128, True),
    (1, 6, 2, 17, 64, True), (2, 4, 1, 64, 64, False),
    # 512 keys and more: the fp16 gradient products (ragged, both head sizes, both masks)
    (1, 4, 1, 1100, 128, True), (1, 2, 2, 777, 64, True), (1, 4, 2, 1090, 128, False),
]


def oracle_full(x, scale, causal, heads=None):
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    return att.backward(q, k, v, do, scale, causal=causal, heads=heads)


def compare_full(gpu, ref, sel_q=(slice(None),), sel_kv=(slice(None),)):
    for name in ("o", "dq"):
        assert_close(name, to_f64(gpu[name])[sel_q], ref[name][sel_q])
    assert_lse(to_f64(gpu["lse"])[sel_q], ref["lse"][sel_q])
    for name in ("dk", "dv"):
        assert_close(name, to_f64(gpu[name])[sel_kv], ref[name][sel_kv])


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}_Hq{}_Hkv{}_S{}_D{}_{}".format(
    *s[:5], "causal" if s[5] else "full"))
def test_small_shapes(shape):
    B, Hq, Hkv, S, D, causal = shape
    say(f"small shape {shape}")
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(100, B, Hq, Hkv, S, D, int(causal)))
    scale = 1.0 / math.sqrt(D)
    gpu = run_gpu(x, causal, scale)
    compare_full(gpu, oracle_full(x, scale, causal))


SHORT_SUBSETS = [  # B, Hq, Hkv, S, D, causal: heads per subset of the one-kernel paths
    (64, 12, 2, 64, 128, True),   # 128 groups, 2 subsets of 3 heads: odd, with partials
    (32, 40, 8, 48, 64, False),   # 256 groups, 1 subset of 5 heads: odd, dK/dV stored directly
    (128, 4, 2, 64, 128, True),   # 256 groups, 1 subset of 2 heads: one pair, stored directly
    # 512 groups: one subset of every head in both kernels; the forward's waves
    # take three heads (six) or three and two (five), so their two Q register
    # sets are reloaded, and the backward runs three pairs
    (64, 48, 8, 64, 128, True),
    (64, 40, 8, 37, 64, False),
]


@pytest.mark.parametrize("shape", SHORT_SUBSETS, ids=lambda s: "B{}_Hq{}_Hkv{}_S{}_D{}_{}".format(
    *s[:5], "causal" if s[5] else "full"))
def test_short_path_head_subsets(shape):
    """The one-kernel backward at 64 tokens or fewer takes a subset's heads in
    pairs, one per group of four waves; with an odd count the second group sits
    out the last pair. With 256 or more (batch, kv head) groups there is one
    subset and dK, dV are stored directly instead of as partials. The
    one-kernel forward gives each wave every other head of its subset, in two
    Q register sets used in turn."""
    B, Hq, Hkv, S, D, causal = shape
    say(f"short-path head subsets {shape}")
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(130, B, Hq, Hkv, S, D, int(causal)))
    scale = 1.0 / math.sqrt(D)
    gpu = run_gpu(x, causal, scale)
    compare_full(gpu, oracle_full(x, scale, causal))


@pytest.mark.parametrize("w", [wl.WORKLOADS[0], wl.WORKLOADS[2]], ids=lambda w: w.name)
def test_workload_full(w):
    """The S=256/D=64 and the batch-16 S=64 workloads, every element."""
    say(f"workload {w.name} full")
    x = wl.workload_inputs(w)
    gpu = run_gpu(x, True, w.scale)
    compare_full(gpu, oracle_full(x, w.scale, True))


def test_workload_llama2_layer_all_groups():
    """S=4096, 64/8 heads: every element of every output (all 8 GQA groups)."""
    w = wl.BY_NAME["llama2_70b_layer_s4096"]
    say(f"workload {w.name}: all 8 groups")
    x = wl.workload_inputs(w)
    gpu = run_gpu(x, True, w.scale)
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    got = {n: to_f64(gpu[n]) for n in ("o", "lse", "dq", "dk", "dv")}
    del gpu
    refs = par.groups_backward(q, k, v, do, w.scale, True, [(0, kvh) for kvh in range(w.Hkv)])
    for n in ("o", "dq"):
        assert_close(n, got[n][0], np.concatenate([r[n] for r in refs]))
    assert_lse(got["lse"][0], np.concatenate([r["lse"] for r in refs]))
    for n in ("dk", "dv"):
        assert_close(n, got[n][0], np.stack([r[n] for r in refs]))


def shift_sums(w, gpu, x):
    """Sanity over every key row: sum_j dK_j = 0 and sum_j dV_j = sum of the group's dO.

    Both are exact consequences of the definition; on bf16 outputs the sums
    carry rounding of order 2^-9 per element, so the bound scales with sqrt(S).
    """
    g = w.group
    dk = to_f64(gpu["dk"]).sum(axis=2)
    dv = to_f64(gpu["dv"]).sum(axis=2)
    do = att.bf16_bits_to_f64(x["do"]).reshape(w.B, w.Hkv, g, w.S, w.D).sum(axis=(2, 3))
    tol = 2e-2 * math.sqrt(w.S)
    assert np.max(np.abs(dk)) <= tol, np.max(np.abs(dk))
    assert np.max(np.abs(dv - do)) <= tol, np.max(np.abs(dv - do))


def test_workload_long_context_whole_group():
    """S=32768 with K x 3: one whole GQA group element by element -- every row of O, LSE
    and dQ of its 4 query heads and every key row of dK, dV of its key/value head --
    plus the shift-invariance sums over all groups."""
    w = wl.BY_NAME["long_context_s32768_k3"]
    kvh = 5
    say(f"workload {w.name}: whole group of kv head {kvh}")
    x = wl.workload_inputs(w)
    gpu = run_gpu(x, True, w.scale)
    g = w.group
    hs = slice(kvh * g, (kvh + 1) * g)
    got = {n: to_f64(gpu[n][0, hs]) for n in ("o", "lse", "dq")}
    got.update({n: to_f64(gpu[n][0, kvh]) for n in ("dk", "dv")})
    shift_sums(w, gpu, x)
    del gpu
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    say(f"workload {w.name}: oracle on the group")
    ref, = par.groups_backward(q, k, v, do, w.scale, True, [(0, kvh)], panel_rows=1024)
    for n in ("o", "dq", "dk", "dv"):
        assert_close(n, got[n], ref[n])
    assert_lse(got["lse"], ref["lse"])


def seeded_blocks(n_blocks, n_total, seed):
    """Block indices: the first, the last and n_blocks - 2 seeded others (sorted, distinct)."""
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, n_total - 1), n_blocks - 2, replace=False)
    return sorted({0, n_total - 1, *(int(i) for i in mid)})


def test_workload_very_long_rows_and_key_blocks():
    """S=81920, 8/1 heads: every row of O, LSE and dQ of all 8 query heads, and dK, dV on
    eight whole 128-key blocks (the first, the last and six seeded ones); the first block
    sees every query row, so it carries the longest accumulation."""
    w = wl.BY_NAME["very_long_s81920"]
    say(f"workload {w.name}: all rows, 8 key blocks")
    x = wl.workload_inputs(w)
    gpu = run_gpu(x, True, w.scale)
    got = {n: to_f64(gpu[n][0]) for n in ("o", "lse", "dq")}
    blocks = seeded_blocks(8, w.S // 128, seed=w.cfg_id)
    cols = np.concatenate([np.arange(128 * j, 128 * j + 128) for j in blocks])
    got.update({n: to_f64(gpu[n][0, 0])[cols] for n in ("dk", "dv")})
    shift_sums(w, gpu, x)
    del gpu
    q, k, v, do = (att.bf16_bits_to_f64(x[n][0]) for n in ("q", "k", "v", "do"))
    say(f"workload {w.name}: oracle rows")
    ref = par.all_rows(q, k[0], v[0], do, w.scale, panel_rows=512)
    for n in ("o", "dq"):
        assert_close(n, got[n], ref[n])
    assert_lse(got["lse"], ref["lse"])
    say(f"workload {w.name}: oracle key blocks {blocks}")
    kb = par.key_blocks_dkdv(q, do, k[0], v[0], ref["lse"], ref["delta"], blocks, 128, w.scale)
    for n, i in (("dk", 0), ("dv", 1)):
        assert_close(f"{n}[blocks]", got[n], np.concatenate([kb[j][i] for j in blocks]))
