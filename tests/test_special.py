"""GPU special cases with closed-form answers, and the C ABI's errors on real tensors.

The expected values here come from the mathematics, not from the oracle:
V = 1 gives O = 1; Q = 0 or scale = 0 gives equal weights, i.e. O_i is the
running mean of V and LSE_i = ln(i + 1); dO = 0 gives zero gradients.
"""
import math

import numpy as np
import pytest

from gpu_helpers import assert_close, assert_lse, run_gpu, say, to_dev, to_f64
from oracle import attention as att
from tiled_attention_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu

ONE_BF16 = 0x3F80


@pytest.mark.parametrize("D", [64, 128])
def test_unit_values_give_unit_output(D):
    say(f"V = 1, D={D}")
    x = wl.make_inputs(1, 4, 2, 300, D, seed=(200, D))
    x["v"] = np.full_like(x["v"], ONE_BF16)
    gpu = run_gpu(x, True, 1.0 / math.sqrt(D))
    o = to_f64(gpu["o"])
    assert np.max(np.abs(o - 1.0)) <= 4e-3, np.max(np.abs(o - 1.0))


@pytest.mark.parametrize("D,mode", [(64, "zero_q"), (128, "zero_q"), (128, "zero_scale")])
def test_equal_weights_give_running_mean(D, mode):
    say(f"equal weights ({mode}), D={D}")
    B, Hq, Hkv, S = 2, 4, 2, 333
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(201, D))
    scale = 1.0 / math.sqrt(D)
    if mode == "zero_q":
        x["q"] = np.zeros_like(x["q"])
    else:
        scale = 0.0
    gpu = run_gpu(x, True, scale)
    v = att.bf16_bits_to_f64(x["v"])
    mean = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    want = np.repeat(mean, Hq // Hkv, axis=1)
    assert_close("o", to_f64(gpu["o"]), want)
    assert_lse(to_f64(gpu["lse"]), np.broadcast_to(np.log(np.arange(1, S + 1)), (B, Hq, S)))


def test_zero_output_gradient_gives_zero_gradients():
    say("dO = 0")
    x = wl.make_inputs(1, 8, 2, 257, 128, seed=(202,))
    x["do"] = np.zeros_like(x["do"])
    gpu = run_gpu(x, True, 1.0 / math.sqrt(128))
    for name in ("dq", "dk", "dv"):
        assert np.all(to_f64(gpu[name]) == 0.0), name


@pytest.mark.parametrize("scale,k_mult,causal", [(-0.2, 1.0, True), (0.5, 3.0, True), (-0.3, 2.0, False)])
def test_unusual_scales_against_oracle(scale, k_mult, causal):
    say(f"scale={scale} k_mult={k_mult} causal={causal}")
    B, Hq, Hkv, S, D = 1, 4, 2, 200, 128
    x = wl.make_inputs(B, Hq, Hkv, S, D, seed=(203, int(1000 * abs(scale)), int(scale < 0), int(causal)), k_mult=k_mult)
    gpu = run_gpu(x, causal, scale)
    q, k, v, do = (att.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = att.backward(q, k, v, do, scale, causal=causal)
    for name in ("o", "dq", "dk", "dv"):
        assert_close(name, to_f64(gpu[name]), ref[name])
    assert_lse(to_f64(gpu["lse"]), ref["lse"])


def test_abi_rejects_misaligned_and_aliased_tensors():
    import torch
    import tiled_attention_memory_amd as tam
    say("ABI errors on device tensors")
    B, Hq, Hkv, S, D = 1, 2, 1, 64, 64
    q = torch.zeros((B, Hq, S, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, S, D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    flat = torch.empty(q.numel() + 1, dtype=torch.bfloat16, device="cuda")
    o_mis = flat[1:].view(B, Hq, S, D)          # contiguous but 2 bytes off alignment
    with pytest.raises(tam.AttnError) as e:
        tam.attn_fwd(q, k, v, o_mis, lse)
    assert e.value.status == 5
    with pytest.raises(tam.AttnError) as e:
        tam.attn_fwd(q, k, v, q, lse)            # o on top of q
    assert e.value.status == 9
    with pytest.raises(TypeError):
        tam.attn_fwd(q.float(), k, v, torch.empty_like(q), lse)
    torch.cuda.synchronize()
