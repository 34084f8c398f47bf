"""Full-mode parity of the two long workloads: every element of every output.

The oracle needs several minutes of host time per workload here, so these
run only when TAM_FULL_PARITY=1 is set (the regular suite checks one whole
GQA group at S = 32768 and all rows plus eight key blocks at S = 81920).
Each prints its error figures per tensor; the results of a run are kept with
the profiles.
"""
import os

import numpy as np
import pytest

import oracle_par as par
from gpu_helpers import assert_close, assert_lse, run_gpu, say, to_f64
from oracle import attention as att
from tiled_attention_memory_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(os.environ.get("TAM_FULL_PARITY") != "1",
                                 reason="full-mode oracle runs only with TAM_FULL_PARITY=1")]


@pytest.mark.parametrize("name,panel", [("long_context_s32768_k3", 1024), ("very_long_s81920", 512)])
def test_long_workload_every_element(name, panel):
    w = wl.BY_NAME[name]
    say(f"full mode {name}")
    x = wl.workload_inputs(w)
    gpu = run_gpu(x, True, w.scale)
    got = {n: to_f64(gpu[n][0]) for n in ("o", "lse", "dq", "dk", "dv")}
    del gpu
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    del x
    for kvh in range(w.Hkv):
        say(f"full mode {name}: group {kvh}")
        ref, = par.groups_backward(q, k, v, do, w.scale, True, [(0, kvh)], panel_rows=panel)
        hs = slice(kvh * w.group, (kvh + 1) * w.group)
        for n in ("o", "dq"):
            assert_close(f"{n}[group {kvh}]", got[n][hs], ref[n])
        assert_lse(got["lse"][hs], ref["lse"])
        for n in ("dk", "dv"):
            assert_close(f"{n}[group {kvh}]", got[n][kvh], ref[n])
