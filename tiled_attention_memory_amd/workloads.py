"""Seeded synthetic workloads for exact causal GQA attention.

This module only describes shapes and draws inputs. It holds none of the
attention arithmetic, so both the CPU oracle's tests and the HIP path can take
their inputs from here without sharing any of the method's code.

Shapes: the five workloads below restate the attention shapes of the pages'
fine-tuning and training runs (Llama-2-70B layer from the FSDP fine-tuning
page, the batch-16 x 64-token LoRA step of the Llama 3.1 405B page, the 32k
context stage of the MI300X MoE training page, and an 80K-token sequence from
the activation/gradient quantisation page). Values are standard normal, as no
real activations are available; the 32k workload scales K by 3 to widen the
softmax range.

Tensors are row-major [B, H, S, D] (D innermost). bf16 values are kept as
their raw 16-bit patterns (numpy uint16) so that no library conversion sits
between the generator and either consumer.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "do": 3}


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    causal: bool = True
    k_mult: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def fwd_flops(self) -> int:
        """Counted forward FLOPs: 4*B*Hq*S^2*D, halved when causal."""
        f = 4 * self.B * self.Hq * self.S * self.S * self.D
        return f // 2 if self.causal else f

    def bwd_flops(self) -> int:
        """Counted backward FLOPs: 2.5x the forward count."""
        return self.fwd_flops() * 5 // 2

    def describe(self) -> dict:
        return {"B": self.B, "Hq": self.Hq, "Hkv": self.Hkv, "S": self.S,
                "D": self.D, "causal": self.causal, "scale": self.scale,
                "k_mult": self.k_mult}


# The five workloads, in the order the headline metric and tests refer to them.
WORKLOADS = [
    Workload(0, "smoke_s256_d64", 1, 4, 4, 256, 64),
    Workload(1, "llama2_70b_layer_s4096", 1, 64, 8, 4096, 128),
    Workload(2, "llama3_405b_lora_b16_s64", 16, 128, 8, 64, 128),
    Workload(3, "long_context_s32768_k3", 1, 32, 8, 32768, 128, k_mult=3.0),
    Workload(4, "very_long_s81920", 1, 8, 1, 81920, 128),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits.

    NaN is not expected from a normal generator and is not special-cased.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # 32-bit sums: a carry out of bit 31 would only reach bit 16 of the shifted
    # value, which the cast to 16 bits drops, so no wider type is needed
    return ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)


def draw(shape, seed, mult: float = 1.0) -> np.ndarray:
    """Standard-normal float32 from PCG64(SeedSequence(seed)), optionally scaled, as bf16 bits."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return f32_to_bf16_bits(x)


def make_inputs(B, Hq, Hkv, S, D, seed=(0,), k_mult=1.0, tensors=("q", "k", "v", "do")):
    """Seeded bf16 inputs: q, do are [B,Hq,S,D]; k, v are [B,Hkv,S,D] (uint16 bit patterns)."""
    out = {}
    for name in tensors:
        h = Hq if name in ("q", "do") else Hkv
        mult = k_mult if name == "k" else 1.0
        out[name] = draw((B, h, S, D), tuple(seed) + (TENSOR_ID[name],), mult)
    return out


def workload_inputs(w: Workload, tensors=("q", "k", "v", "do")):
    """Inputs of a named workload, seeded by its id."""
    return make_inputs(w.B, w.Hq, w.Hkv, w.S, w.D, seed=(w.cfg_id,), k_mult=w.k_mult,
                       tensors=tensors)
