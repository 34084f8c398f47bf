#!/usr/bin/env python3
"""Headline benchmark: exact causal GQA attention, forward + backward, on one MI355X.

One step = attn_fwd then attn_bwd (every kernel of the path) on one batch of
seeded synthetic inputs that are already resident in HBM. Default workload:
the Llama-2-70B attention layer shape, B=1, Hq=64, Hkv=8, S=4096, D=128,
bf16, scale 1/sqrt(128).

Throughput counts 4*B*Hq*S^2*D FLOPs for the forward pass and 2.5x that for
the backward pass, halved for the causal mask. Per-kernel durations come from
HIP events recorded on the launch stream around every kernel of every timed
step. Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 bf16 flop/clk x 2.4 GHz (AMD's 2.5 PFLOP/s dense figure)
PEAK_HBM_GBS = 8000.0       # HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_{workload}.json")
KERNEL_SOURCES = ["attn_device.h", "attn_launch.h", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_short.hip"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the timing needs (the runtime torch already loaded)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL)
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def check(self, err, what):
        if err != 0:
            raise RuntimeError(f"{what} failed with HIP error {err}")

    def event(self):
        e = ctypes.c_void_p()
        self.check(self.lib.hipEventCreate(ctypes.byref(e)), "hipEventCreate")
        return e.value

    def record(self, ev, stream):
        self.check(self.lib.hipEventRecord(ev, stream), "hipEventRecord")

    def ms(self, a, b):
        out = ctypes.c_float()
        self.check(self.lib.hipEventElapsedTime(ctypes.byref(out), a, b), "hipEventElapsedTime")
        return float(out.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)

    def attribute(self, attr, device=0):
        out = ctypes.c_int()
        self.check(self.lib.hipDeviceGetAttribute(ctypes.byref(out), attr, device), "hipDeviceGetAttribute")
        return out.value


# hipDeviceAttribute_t values (hip_runtime_api.h)
HIP_ATTR_CLOCK_RATE_KHZ = 5
HIP_ATTR_MEMORY_CLOCK_RATE_KHZ = 60
HIP_ATTR_MULTIPROCESSOR_COUNT = 63


def device_facts(hip):
    """CU count and peak engine clock as the runtime reports them, and the bf16 dense peak they imply
    (4096 flop per clock per CU on gfx950)."""
    import torch
    props = torch.cuda.get_device_properties(0)
    cus = hip.attribute(HIP_ATTR_MULTIPROCESSOR_COUNT)
    sclk_mhz = hip.attribute(HIP_ATTR_CLOCK_RATE_KHZ) / 1e3
    return {"name": props.name, "arch": props.gcnArchName, "cus": cus, "max_sclk_mhz": sclk_mhz,
            "max_mclk_mhz": hip.attribute(HIP_ATTR_MEMORY_CLOCK_RATE_KHZ) / 1e3,
            "bf16_peak_at_max_sclk_tflops": round(cus * 4096 * sclk_mhz * 1e6 / 1e12, 1)}


def hbm_probe(hip, mib, reps=20, flush=None, flush_mode="read"):
    """Achievable HBM bandwidth with plain library kernels on buffers of `mib` MiB: sequential
    write (fill), read (sum), copy, and a gather of random 4 KiB blocks. GB/s = bytes moved over
    the median event time of `reps` runs after two warm-up runs. With `flush` (a device buffer)
    each timed run starts after the buffer is read (or overwritten), outside the events, so that
    small buffers are timed from HBM rather than from the caches."""
    import torch
    n = (mib << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    rows = a.view(-1, 1024)                     # 4 KiB rows
    g = torch.Generator(device="cuda").manual_seed(1)
    idx = torch.randperm(rows.shape[0], device="cuda", generator=g)[: rows.shape[0] // 2]
    out_rows = torch.empty((idx.numel(), 1024), dtype=torch.float32, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    size = a.numel() * 4
    cases = {
        "write": (lambda: a.fill_(2.0), size),
        "read": (lambda: a.sum(), size),
        "copy": (lambda: b.copy_(a), 2 * size),
        "gather_4k_random": (lambda: torch.index_select(rows, 0, idx, out=out_rows), 2 * idx.numel() * 4096),
    }
    res = {}
    for name, (fn, nbytes) in cases.items():
        for _ in range(2):
            fn()
        times = []
        for i in range(reps):
            if flush is not None:
                if flush_mode == "write":
                    flush.fill_(float(i))
                else:
                    flush.sum()
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, sh)
            fn()
            hip.record(e1, sh)
            torch.cuda.synchronize()
            times.append(hip.ms(e0, e1))
            hip.destroy(e0)
            hip.destroy(e1)
        times.sort()
        med = times[len(times) // 2]
        res[name] = {"bytes": nbytes, "ms_median": round(med, 4), "gbps": round(nbytes / (med * 1e-3) / 1e9, 1)}
    return res


def kernel_source_sha():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tiled_attention_memory_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE.format(workload=workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(kernel)
    if not rec or rec.get("workload") != workload or rec.get("source_sha") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def alg_bytes(w):
    """Bytes the method itself must move, each tensor once: forward reads Q, K, V and
    writes O and LSE; backward reads Q, K, V, O, dO and LSE, writes Delta once and
    reads it twice, and writes dQ, dK and dV."""
    q = w.B * w.Hq * w.S * w.D * 2
    kv = w.B * w.Hkv * w.S * w.D * 2
    rows = w.B * w.Hq * w.S * 4
    fwd = q + 2 * kv + q + rows
    bwd = 3 * q + 2 * kv + rows + 3 * rows + q + 2 * kv
    return fwd, bwd


def cpu_baseline(w, x, n_groups):
    """The fp64 oracle, untuned, on a bounded sample: whole GQA groups of the same workload."""
    import numpy as np
    from oracle import attention as att
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    groups = [(0, g) for g in range(n_groups)]
    t0 = time.perf_counter()
    att.backward(q, k, v, do, w.scale, causal=True, heads=groups)
    dt = time.perf_counter() - t0
    heads = n_groups * w.group
    flops = (w.fwd_flops() + w.bwd_flops()) * heads / (w.B * w.Hq)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle, forward+backward of {n_groups} of the {w.B * w.Hkv} GQA "
                      f"groups ({heads} of {w.B * w.Hq} query heads) of the same workload, "
                      f"{dt:.1f} s wall; counted FLOPs of that sample"}


def cp_bench(args, w):
    """One rank of an N-way context-parallel split on this GPU: the last query block
    (the heaviest under a causal mask) against all N key blocks, through the block
    calls. Counted FLOPs are those of the rank's visible (query, key) pairs, with the
    same forward and 2.5x backward factors as the whole-sequence metric."""
    import numpy as np
    import torch
    import tiled_attention_memory_amd as tam
    from tiled_attention_memory_amd import workloads as wl
    n = args.cp
    if w.S % n:
        print(f"--cp {n} must divide S = {w.S}", file=sys.stderr)
        sys.exit(2)
    s = w.S // n
    r = n - 1
    x = wl.workload_inputs(w)
    dev = {k_: torch.from_numpy(np.ascontiguousarray(x[k_]).view(np.int16)).view(torch.bfloat16).cuda()
           for k_ in x}
    q0 = r * s
    qb = dev["q"][:, :, q0:q0 + s].contiguous()
    dob = dev["do"][:, :, q0:q0 + s].contiguous()
    kbs = [(dev["k"][:, :, b * s:(b + 1) * s].contiguous(), dev["v"][:, :, b * s:(b + 1) * s].contiguous())
           for b in range(n)]
    del dev
    parts = [(torch.empty((w.B, w.Hq, s, w.D), dtype=torch.float32, device="cuda"),
              torch.empty((w.B, w.Hq, s), dtype=torch.float32, device="cuda")) for _ in range(n)]
    o = torch.empty_like(qb)
    lse = torch.empty((w.B, w.Hq, s), dtype=torch.float32, device="cuda")
    ws = torch.empty(tam.attn_bwd_block_workspace_bytes(w.B, w.Hq, w.Hkv, s, s, w.D), dtype=torch.uint8,
                     device="cuda")
    dq = torch.empty_like(qb)
    dks = [(torch.empty_like(kk), torch.empty_like(vv)) for kk, vv in kbs]
    hip = Hip()
    sh = torch.cuda.current_stream().cuda_stream

    def step(ev=None):
        if ev:
            hip.record(ev[0], sh)
        for b, (kk, vv) in enumerate(kbs):
            tam.attn_fwd_block(qb, kk, vv, parts[b][0], parts[b][1], q0, b * s, causal=True, scale=w.scale)
        tam.attn_merge([p[0] for p in parts], [p[1] for p in parts], o, lse)
        if ev:
            hip.record(ev[1], sh)
        tam.attn_bwd_block_begin(o, dob, lse, ws, w.Hkv, s)
        for b, (kk, vv) in enumerate(kbs):
            tam.attn_bwd_block_dq(qb, kk, vv, dob, ws, q0, b * s, causal=True, scale=w.scale)
        tam.attn_bwd_block_dq_end(dq, ws, w.Hkv, s, scale=w.scale)
        for b, (kk, vv) in enumerate(kbs):
            tam.attn_bwd_block_dkdv(qb, kk, vv, dob, dks[b][0], dks[b][1], ws, q0, b * s, causal=True,
                                    scale=w.scale)
        if ev:
            hip.record(ev[2], sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [(hip.event(), hip.event(), hip.event()) for _ in range(K)]
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    fwd_ms = sum(hip.ms(e[0], e[1]) for e in evs) / K
    bwd_ms = sum(hip.ms(e[1], e[2]) for e in evs) / K
    for e in evs:
        for h in e:
            hip.destroy(h)
    pairs = r * s * s + s * (s + 1) // 2            # visible (query, key) pairs of the rank, per head
    fwd_flops = 4 * w.B * w.Hq * w.D * pairs
    bwd_flops = 5 * fwd_flops // 2
    ms_step = fwd_ms + bwd_ms
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    out = {
        "metric": f"attention fwd+bwd TFLOP/s, one rank of a {n}-way context-parallel split (block calls)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}_cp{n}_rank{r}", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S,
                   "D": w.D, "block": s, "causal": True},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 1),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 1),
    }
    print(json.dumps(out), flush=True)


def decode_bench(args, w):
    """attn_decode on a synthetic cache (seeded N(0,1), like the training shapes).

    Bound by HBM: the algorithmic bytes are the cache (K and V) read once plus the
    new tokens' Q read and O, LSE written; value is those bytes over the call's time."""
    import numpy as np
    import torch
    import tiled_attention_memory_amd as tam
    from tiled_attention_memory_amd import workloads as wl
    B, Sq, Sk = (int(t) for t in args.decode.split(","))
    # the cache (Sk keys and values) and the Sq new tokens' queries
    x = wl.make_inputs(B, w.Hq, w.Hkv, Sk, w.D, seed=(500, B, Sq, Sk), tensors=("k", "v"))
    x.update(wl.make_inputs(B, w.Hq, w.Hkv, Sq, w.D, seed=(501, B, Sq, Sk), tensors=("q",)))
    dev = {n: torch.from_numpy(np.ascontiguousarray(x[n]).view(np.int16)).view(torch.bfloat16).cuda()
           for n in ("q", "k", "v")}
    del x
    q, k, v = dev["q"], dev["k"], dev["v"]
    del dev
    o = torch.empty_like(q)
    lse = torch.empty((B, w.Hq, Sq), dtype=torch.float32, device="cuda")
    ws = torch.empty(tam.attn_decode_workspace_bytes(B, w.Hq, w.Hkv, Sq, Sk, w.D), dtype=torch.uint8,
                     device="cuda")
    flush = (torch.empty(args.flush_mib << 18, dtype=torch.float32, device="cuda") if args.flush_mib else None)
    hip = Hip()
    sh = torch.cuda.current_stream().cuda_stream
    for _ in range(args.warmup):
        tam.attn_decode(q, k, v, o, lse, ws, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    K = args.steps
    evs = [(hip.event(), hip.event()) for _ in range(K)]
    if flush is not None:
        flush.fill_(1.0)
    for i in range(K):
        if flush is not None:
            # reading evicts the cache without leaving dirty lines whose write-back
            # would compete with the timed call; --flush-mode write measures that case
            if args.flush_mode == "write":
                flush.fill_(float(i))
            else:
                flush.sum()
        hip.record(evs[i][0], sh)
        tam.attn_decode(q, k, v, o, lse, ws, causal=True, scale=w.scale)
        hip.record(evs[i][1], sh)
    torch.cuda.synchronize()
    ms = sum(hip.ms(a, b) for a, b in evs) / K
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    cache = 2 * B * w.Hkv * Sk * w.D * 2
    qo = 2 * B * w.Hq * Sq * w.D * 2 + B * w.Hq * Sq * 4
    gbps = (cache + qo) / (ms * 1e-3) / 1e9
    out = {
        "metric": "attention decode GB/s (algorithmic bytes: cache read once, new tokens in and out)",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode_b{B}_q{Sq}_s{Sk}_h{w.Hq}x{w.Hkv}_d{w.D}", "B": B, "Hq": w.Hq,
                   "Hkv": w.Hkv, "Sq": Sq, "Sk": Sk, "D": w.D, "causal": True,
                   "cache": ("warm" if flush is None else "cold" if args.flush_mode == "read"
                             else "cold, after a write")},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBS, 4), "traffic": None},
    }
    print(json.dumps(out), flush=True)


# Whole-sequence calls of at most this many tokens (without dropout or rotation)
# take the library's one-kernel backward.
SHORT_MAX = 64


def short_path(w, option=None):
    return w.S <= SHORT_MAX and not option


def kernel_flops(w):
    """Algorithmic and executed FLOPs per launch of each kernel of the step.

    Algorithmic: the share of the counted total each kernel carries out -- the
    forward kernel's two products; the dK/dV kernel's recomputed S and dP plus
    dV and dK; the dQ kernel's dQ product. Executed adds the dQ kernel's second
    recomputation of S and dP and its exact-Delta correction product, and, on
    the bf16 path, the lo halves of the split operands (dV, dK, dQ). The
    library takes the fp16 path (one product per gradient) for whole-sequence
    calls over 512 keys or more. Short sequences take one backward kernel that
    carries the whole counted backward and executes S, dP and the hi and lo
    halves of dV, dK and dQ.
    """
    if short_path(w):
        return ({"attn_fwd_short_kernel": w.fwd_flops(), "attn_bwd_short_kernel": w.bwd_flops()},
                {"attn_fwd_short_kernel": w.fwd_flops(), "attn_bwd_short_kernel": 4 * w.fwd_flops()})
    fp16_path = w.S >= 512
    alg = {
        "attn_fwd_kernel": w.fwd_flops(),
        "attn_bwd_dkdv_kernel": 2 * w.fwd_flops(),
        "attn_bwd_dq_kernel": w.fwd_flops() // 2,
    }
    exe = {
        "attn_fwd_kernel": w.fwd_flops(),
        "attn_bwd_dkdv_kernel": (2 if fp16_path else 3) * w.fwd_flops(),
        "attn_bwd_dq_kernel": (4 if fp16_path else 5) * w.fwd_flops() // 2,
    }
    return alg, exe


def short_kernel_bytes(w):
    """Algorithmic bytes of the one-kernel paths, each tensor they must touch once: the
    forward reads Q, K, V and writes O, LSE; the backward reads Q, K, V, dO, LSE and
    writes dQ, dK, dV (it needs neither O nor a Delta round trip)."""
    q = w.B * w.Hq * w.S * w.D * 2
    kv = w.B * w.Hkv * w.S * w.D * 2
    rows = w.B * w.Hq * w.S * 4
    return {"attn_fwd_short_kernel": 2 * q + 2 * kv + rows,
            "attn_bwd_short_kernel": 3 * q + 4 * kv + rows}


def bwd_products(w):
    """Operand precision of the backward's matrix products for this workload."""
    if w.S >= 512:
        return ("fp16 operands with power-of-two block scales (every dK/dV product; S, P K and dQ "
                "of the dQ kernel), bf16 dP in the dQ kernel; fp32 accumulation")
    return ("bf16 operands, P and dS as hi + lo bf16 pairs; fp32 accumulation"
            + (" (one backward kernel)" if short_path(w) else ""))


def summarize(w, per, bwd_ms, ms_step, steps_ms, K, warmup, option=None, dropout=0.0, rope=0.0,
              traffic=measured_traffic):
    """The bench line from measured times (ms): per-kernel averages `per`, the backward
    pass `bwd_ms`, the step `ms_step` and the sorted per-step times `steps_ms`."""
    flops = w.fwd_flops() + w.bwd_flops()
    value = flops / (ms_step * 1e-3) / 1e12
    alg_flops, exec_flops = kernel_flops(w)
    fwd_ms = per["attn_fwd_kernel"]
    if option:
        # the option entry points take no events between their kernels: report
        # the forward call and the whole backward call
        per = {"attn_fwd_kernel": fwd_ms, "backward_pass": bwd_ms}
    elif short_path(w):
        per = {("attn_fwd_short_kernel" if n == "attn_fwd_kernel" else n): t for n, t in per.items()}
    kernels = {}
    for name, t in per.items():
        rec = {"ms": round(t, 4)}
        if name in alg_flops and t > 0:
            rec["alg_tflops"] = round(alg_flops[name] / (t * 1e-3) / 1e12, 1)
            rec["exec_tflops"] = round(exec_flops[name] / (t * 1e-3) / 1e12, 1)
        kernels[name] = rec
    dominant = max((n for n in alg_flops if n in per), key=lambda n: per[n])
    if short_path(w, option):
        # one key tile per row: a few products per byte, so the bound is HBM
        ach = short_kernel_bytes(w)[dominant] / (per[dominant] * 1e-3) / 1e9
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic(dominant, w.name)}
    else:
        ach = alg_flops[dominant] / (per[dominant] * 1e-3) / 1e12
        ach_exec = exec_flops[dominant] / (per[dominant] * 1e-3) / 1e12
        roofline = {"kernel": dominant, "bound": "mfma", "achieved": round(ach, 1),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": None if option else traffic(dominant, w.name),
                    # the products the kernel executes, recomputations included
                    "exec_achieved": round(ach_exec, 1), "exec_frac": round(ach_exec / PEAK_BF16_TFLOPS, 4)}
    fb, bb = alg_bytes(w)
    return {
        "metric": "attention fwd+bwd TFLOP/s and % of bf16 MFMA peak, causal S=4096 D=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # inputs and outputs are bf16 (LSE fp32); bwd_products gives the backward's operands
        "dtype": "bf16",
        "bwd_products": bwd_products(w),
        "data": "synthetic",
        "config": {"workload": w.name + (f"_dropout{dropout:g}" if dropout else "")
                   + (f"_rope{rope:g}" if rope else ""), "B": w.B,
                   "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "D": w.D, "causal": True, "global_batch": w.B,
                   "seq_len": w.S, "parallelism": "none", **({"dropout": dropout} if dropout else {}),
                   **({"rope_base": rope} if rope else {})},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "ms_step_median": round(steps_ms[len(steps_ms) // 2], 4),
        "ms_step_min": round(steps_ms[0], 4),
        "fwd_tflops": round(w.fwd_flops() / (fwd_ms * 1e-3) / 1e12, 1),
        "bwd_tflops": round(w.bwd_flops() / (bwd_ms * 1e-3) / 1e12, 1),
        # algorithmic bytes (each tensor once) over the pass time, for the short shapes
        "fwd_alg_gbps": round(fb / (fwd_ms * 1e-3) / 1e9, 1),
        "bwd_alg_gbps": round(bb / (bwd_ms * 1e-3) / 1e9, 1),
        "kernels": kernels,
        "roofline": roofline,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama2_70b_layer_s4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cp", type=int, default=0, metavar="N",
                    help="instead of the whole-sequence step, time the last rank of an N-way "
                         "context-parallel split of the workload: its query block against every key "
                         "block (forward block calls + merge, then the block backward protocol)")
    ap.add_argument("--decode", default="", metavar="B,SQ,SK",
                    help="instead of the training step, time attn_decode: B sequences with SQ new tokens "
                         "per head against an SK-key cache, with the workload's heads and head size")
    ap.add_argument("--dropout", type=float, default=0.0, metavar="P",
                    help="run the step with dropout probability P on the probabilities "
                         "(attn_fwd_dropout / attn_bwd_dropout); the headline runs without")
    ap.add_argument("--rope", type=float, default=0.0, metavar="BASE",
                    help="run the step with rotary position embedding of this base on Q and K "
                         "(attn_fwd_rope / attn_bwd_rope); the headline runs without")
    ap.add_argument("--flush-mib", type=int, default=0, metavar="MIB",
                    help="before each step, overwrite a MIB-mebibyte buffer so that L2 and the "
                         "memory-side cache start cold (for the short, bandwidth-bound shapes); "
                         "the step time is then the sum of the per-kernel event times")
    ap.add_argument("--flush-mode", choices=("read", "write"), default="read",
                    help="with --flush-mib: evict the cache by reading the buffer (default) or by "
                         "overwriting it, which leaves dirty lines whose write-back overlaps the "
                         "timed call")
    ap.add_argument("--cpu-groups", type=int, default=8)
    ap.add_argument("--hbm-probe", type=int, default=0, metavar="MIB",
                    help="instead of attention: achievable HBM bandwidth of plain library kernels "
                         "(fill, sum, copy, random 4 KiB gather) on MIB-sized buffers")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, copy a MIB-mebibyte device buffer 3 times (a plain copy "
                         "kernel of known size, to scale rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the attention path shards by independent (batch, kv-head) "
              f"groups with no exchange, and this build runs on a single MI355X; --gpus {args.gpus} "
              f"is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import tiled_attention_memory_amd as tam
    from tiled_attention_memory_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tam.load()  # fail loudly if the HIP library is missing
    if args.hbm_probe:
        hip = Hip()
        flush = (torch.empty(args.flush_mib << 18, dtype=torch.float32, device="cuda")
                 if args.flush_mib else None)
        res = hbm_probe(hip, args.hbm_probe, flush=flush, flush_mode=args.flush_mode)
        cache = "warm" if flush is None else "cold" if args.flush_mode == "read" else "cold, after a write"
        print(json.dumps({"metric": "achievable HBM bandwidth of library kernels", "value": res["copy"]["gbps"],
                          "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "peak_gbps": 8000.0,
                          "buffer_mib": args.hbm_probe, "cache": cache, "probes": res,
                          "device": device_facts(hip)}))
        return
    w = wl.BY_NAME[args.workload]
    log(f"[bench] workload {w.name}: {w.describe()}")
    if args.cp:
        return cp_bench(args, w)
    if args.decode:
        return decode_bench(args, w)
    x = wl.workload_inputs(w)
    dev = {n: torch.from_numpy(np.ascontiguousarray(x[n]).view(np.int16)).view(torch.bfloat16).cuda()
           for n in x}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = tam.rope_workspace_for(q, k) if args.rope else tam.workspace_for(q, k)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(ev_f=None, ev_b=None):
        if ev_f:
            hip.record(ev_f[0], sh)
        if args.rope:
            tam.attn_fwd_rope(q, k, v, o, lse, ws, args.rope, causal=True, scale=w.scale, stream=stream)
        elif args.dropout:
            tam.attn_fwd_dropout(q, k, v, o, lse, args.dropout, 1234, causal=True, scale=w.scale, stream=stream)
        else:
            tam.attn_fwd(q, k, v, o, lse, causal=True, scale=w.scale, stream=stream)
        if ev_f:
            hip.record(ev_f[1], sh)
        if args.dropout or args.rope:
            # no per-kernel events on these paths: the whole backward pass is bracketed instead
            if ev_b:
                hip.record(ev_b[0], sh)
            if args.rope:
                tam.attn_bwd_rope(q, k, v, o, do, lse, dq, dk, dv, ws, args.rope, causal=True, scale=w.scale,
                                  stream=stream)
            else:
                tam.attn_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, ws, args.dropout, 1234, causal=True,
                                     scale=w.scale, stream=stream)
            if ev_b:
                for i in range(1, tam.BWD_EVENTS):
                    hip.record(ev_b[i], sh)
        else:
            tam.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True, scale=w.scale,
                         stream=stream, events=ev_b)

    hip = Hip()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev_f = [(hip.event(), hip.event()) for _ in range(K)]
    ev_b = [(ctypes.c_void_p * tam.BWD_EVENTS)(*[hip.event() for _ in range(tam.BWD_EVENTS)])
            for _ in range(K)]
    e0, e1 = hip.event(), hip.event()
    flush = (torch.empty(args.flush_mib << 18, dtype=torch.float32, device="cuda")
             if args.flush_mib else None)
    log(f"[bench] {args.warmup} warmup steps done; timing {K} steps")
    # Pass 1, the step time: K steps with events only around the whole run (an
    # event recorded between two kernels costs about 3 us of stream time), or,
    # with flushing, around each step, so that the fills stay outside.
    ev_s = [(hip.event(), hip.event()) for _ in range(K)] if flush is not None else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(e0, sh)
    def evict(i):
        # reading evicts the cache without leaving dirty lines whose write-back
        # would compete with the timed step; --flush-mode write measures that case
        if args.flush_mode == "write":
            flush.fill_(float(i))
        else:
            flush.sum()

    if flush is not None:
        flush.fill_(1.0)
    for i in range(K):
        if flush is not None:
            evict(i)
            hip.record(ev_s[i][0], sh)
        step()
        if flush is not None:
            hip.record(ev_s[i][1], sh)
    hip.record(e1, sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = hip.ms(e0, e1)
    # Pass 2, the breakdown: the same K steps again with events around every kernel.
    log(f"[bench] timing {K} more steps with per-kernel events")
    for i in range(K):
        if flush is not None:
            evict(i)
        step(ev_f[i], ev_b[i])
    torch.cuda.synchronize()

    def avg(pairs):
        return sum(hip.ms(a, b) for a, b in pairs) / len(pairs)

    # per-step times of pass 2, forward start to backward end
    # per-step times, forward start to backward end: pass 1's with flushing, else pass 2's
    steps_ms = sorted(hip.ms(*ev_s[i]) if flush is not None else hip.ms(ev_f[i][0], ev_b[i][tam.BWD_EVENTS - 1])
                      for i in range(K))

    option = "dropout" if args.dropout else "rope" if args.rope else None
    if short_path(w, option):
        # the one-kernel backward lies between events 0 and 1, its partials' sum between 3 and 4
        per = {
            "attn_fwd_kernel": avg(ev_f),
            "attn_bwd_short_kernel": avg([(e[0], e[1]) for e in ev_b]),
            "attn_bwd_reduce_kernel": avg([(e[3], e[4]) for e in ev_b]),
        }
    else:
        per = {
            "attn_fwd_kernel": avg(ev_f),
            "attn_bwd_dq_kernel": avg([(e[1], e[2]) for e in ev_b]),
            "attn_bwd_dkdv_kernel": avg([(e[2], e[3]) for e in ev_b]),
            "attn_bwd_reduce_kernel": avg([(e[3], e[4]) for e in ev_b]),
        }
    ms_step = total_ms / K if flush is None else avg(ev_s)
    # The backward's share of the step: the step (pass 1, no events between the
    # kernels) less the forward kernel. Pass 2's bracket of the backward would
    # also hold the cost of the events recorded inside it.
    bwd_ms = ms_step - per["attn_fwd_kernel"]
    for pair in ev_f + (ev_s or []):
        for e in pair:
            hip.destroy(e)
    for e in ev_b:
        for j in range(tam.BWD_EVENTS):
            hip.destroy(e[j])

    out = summarize(w, per, bwd_ms, ms_step, steps_ms, K, args.warmup, option=option, dropout=args.dropout,
                    rope=args.rope)
    out["config"]["cache"] = ("warm" if flush is None else "cold" if args.flush_mode == "read"
                              else "cold, after a write")
    out["device"] = device_facts(hip)
    log(f"[bench] {K} steps: {ms_step:.4f} ms/step (events), wall {wall / K * 1e3:.4f} ms/step; "
        f"kernels {out['kernels']}")
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n * 4
        del src, dst
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_groups)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
