"""bench.py's harness on the CPU: counted FLOPs, algorithmic bytes, the fields and
derivations of its JSON line from recorded timings, the CPU-baseline record, and
the one-GPU guard. Nothing here touches a GPU.
"""
import json
import os
import subprocess
import sys

import pytest

import bench
from tiled_attention_memory_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Exact counted FLOPs of the five workloads: forward 4*B*Hq*S^2*D/2 (causal),
# backward 2.5x that.
APPENDIX_B = {
    "smoke_s256_d64": (33_554_432, 83_886_080),
    "llama2_70b_layer_s4096": (274_877_906_944, 687_194_767_360),
    "llama3_405b_lora_b16_s64": (2_147_483_648, 5_368_709_120),
    "long_context_s32768_k3": (8_796_093_022_208, 21_990_232_555_520),
    "very_long_s81920": (13_743_895_347_200, 34_359_738_368_000),
}

# Per-kernel event averages (ms) of a recorded headline run.
RECORDED = {"attn_fwd_kernel": 0.2599, "attn_bwd_dq_kernel": 0.5493, "attn_bwd_dkdv_kernel": 0.5327,
            "attn_bwd_reduce_kernel": 0.0156}


@pytest.mark.parametrize("name", list(APPENDIX_B))
def test_counted_flops(name):
    w = wl.BY_NAME[name]
    assert (w.fwd_flops(), w.bwd_flops()) == APPENDIX_B[name]
    assert w.fwd_flops() == 2 * w.B * w.Hq * w.S * w.S * w.D


def test_algorithmic_bytes():
    """Forward: Q, K, V in, O, LSE out; backward: Q, K, V, O, dO, LSE in, Delta written
    once and read twice, dQ, dK, dV out (MB = 1e6 bytes)."""
    fb, bb = bench.alg_bytes(wl.BY_NAME["llama2_70b_layer_s4096"])
    assert round(fb / 1e6, 1) == 152.0 and round(bb / 1e6, 1) == 306.2
    fb, bb = bench.alg_bytes(wl.BY_NAME["llama3_405b_lora_b16_s64"])
    assert round(fb / 1e6, 1) == 71.8 and round(bb / 1e6, 1) == 144.7


def test_kernel_flops_cover_the_counted_total():
    """The algorithmic shares of the forward, dK/dV and dQ kernels add up to the counted
    forward + backward FLOPs."""
    for w in wl.WORKLOADS:
        alg, exe = bench.kernel_flops(w)
        assert sum(alg.values()) == w.fwd_flops() + w.bwd_flops()
        for n in alg:
            assert exe[n] >= alg[n]


def test_line_from_recorded_timings():
    w = wl.BY_NAME["llama2_70b_layer_s4096"]
    bwd_ms = sum(v for k, v in RECORDED.items() if k != "attn_fwd_kernel")
    ms_step = 1.4193
    steps = sorted([1.3687, 1.3631, 1.37, 1.40])
    out = bench.summarize(w, dict(RECORDED), bwd_ms, ms_step, steps, K=20, warmup=5,
                          traffic=lambda kernel, workload: 123)
    json.dumps(out)
    for key, val in (("unit", "TFLOP/s"), ("n_gpus", 1), ("steps", 20), ("warmup", 5),
                     ("higher_is_better", True), ("scaling", "weak"), ("vs_baseline", None),
                     ("dtype", "bf16"), ("data", "synthetic")):
        assert out[key] == val, key
    assert out["metric"] == "attention fwd+bwd TFLOP/s and % of bf16 MFMA peak, causal S=4096 D=128"
    assert out["config"]["workload"] == w.name and out["config"]["S"] == 4096
    counted = sum(APPENDIX_B[w.name])
    assert out["value"] == round(counted / (ms_step * 1e-3) / 1e12, 2)
    assert out["pct_of_peak"] == round(100 * out["value"] / 2516.6, 2)
    assert out["ms_step_median"] == 1.37 and out["ms_step_min"] == 1.3631
    assert out["fwd_tflops"] == round(APPENDIX_B[w.name][0] / 0.2599e-3 / 1e12, 1)
    assert out["bwd_tflops"] == round(APPENDIX_B[w.name][1] / (bwd_ms * 1e-3) / 1e12, 1)
    assert "fp16" in out["bwd_products"]
    r = out["roofline"]
    # the dominant kernel is the longest one; its algorithmic share is the dQ product
    assert r["kernel"] == "attn_bwd_dq_kernel" and r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["peak"] == 2516.6
    ach = APPENDIX_B[w.name][0] / 2 / 0.5493e-3 / 1e12
    assert r["achieved"] == round(ach, 1) and r["frac"] == round(ach / 2516.6, 4)
    assert r["exec_achieved"] == round(4 * ach, 1)
    assert r["traffic"] == 123


def test_line_with_an_option_reports_the_backward_call():
    w = wl.BY_NAME["llama2_70b_layer_s4096"]
    out = bench.summarize(w, dict(RECORDED), 1.2, 1.5, [1.5], K=1, warmup=0, option="dropout", dropout=0.1)
    assert set(out["kernels"]) == {"attn_fwd_kernel", "backward_pass"}
    assert out["roofline"]["kernel"] == "attn_fwd_kernel" and out["roofline"]["traffic"] is None
    assert out["config"]["workload"].endswith("_dropout0.1")


def test_short_sequences_report_the_bf16_products():
    assert "hi + lo" in bench.bwd_products(wl.BY_NAME["llama3_405b_lora_b16_s64"])


def test_short_sequences_take_the_one_kernel_backward():
    """Up to 64 tokens the backward is one kernel: it carries the whole counted backward
    and executes S, dP and both halves of dV, dK and dQ (8 products of fwd/2 each)."""
    w = wl.BY_NAME["llama3_405b_lora_b16_s64"]
    alg, exe = bench.kernel_flops(w)
    assert set(alg) == {"attn_fwd_short_kernel", "attn_bwd_short_kernel"}
    assert alg["attn_bwd_short_kernel"] == w.bwd_flops() and exe["attn_bwd_short_kernel"] == 4 * w.fwd_flops()
    assert "one backward kernel" in bench.bwd_products(w)
    assert not bench.short_path(w, option="dropout")
    # bytes each one-kernel pass must touch (MB = 1e6): fwd Q, K, V in, O, LSE out;
    # bwd Q, K, V, dO, LSE in, dQ, dK, dV out
    b = bench.short_kernel_bytes(w)
    assert round(b["attn_fwd_short_kernel"] / 1e6, 1) == 71.8 and round(b["attn_bwd_short_kernel"] / 1e6, 1) == 109.6
    per = {"attn_fwd_kernel": 0.02, "attn_bwd_short_kernel": 0.03, "attn_bwd_reduce_kernel": 0.005}
    out = bench.summarize(w, per, 0.04, 0.06, [0.06], K=1, warmup=0, traffic=lambda kernel, workload: 7)
    assert set(out["kernels"]) == {"attn_fwd_short_kernel", "attn_bwd_short_kernel", "attn_bwd_reduce_kernel"}
    r = out["roofline"]
    assert r["kernel"] == "attn_bwd_short_kernel" and r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == round(b["attn_bwd_short_kernel"] / 0.03e-3 / 1e9, 1) and r["peak"] == 8000
    assert r["traffic"] == 7
    assert out["bwd_alg_gbps"] == round(bench.alg_bytes(w)[1] / 0.04e-3 / 1e9, 1)
    assert out["fwd_alg_gbps"] == round(bench.alg_bytes(w)[0] / 0.02e-3 / 1e9, 1)


def test_cpu_baseline_record():
    w = wl.WORKLOADS[0]
    x = wl.workload_inputs(w)
    rec = bench.cpu_baseline(w, x, 1)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert isinstance(rec["cores"], int) and rec["cores"] >= 1
    assert rec["value"] > 0 and "1 of the 4 GQA groups" in rec["sample"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
