"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and quantises them to the input dtypes; it
holds none of the projection or reduction arithmetic. Both the HIP path and
the CPU oracle receive exactly the arrays produced here.

Recipe (no trained weights or datasets are involved):
  * weights ~ N(0, 0.02) (0.02 read as the standard deviation), sampled in
    float64, rounded to float32, then to bf16 nearest-even;
  * activations x and expert inputs u ~ N(0, 1) -> bf16 the same way;
  * residual stream and routing logits ~ N(0, 1) float32;
  * the other ranks' partials, which a real run would receive over the
    wire, ~ N(0, 0.02 * sqrt(K_r)) float32, the spread of a real partial.
Each tensor has its own substream keyed by (seed, workload, layer, tensor,
rank), so a tensor's bytes do not depend on which other tensors are drawn.

Host arrays come from numpy's PCG64. Large device tensors (benchmark sizes)
come from torch's seeded device generator instead; tests that check such a
tensor against the oracle copy the sampled part back to the host.
"""
from __future__ import annotations

import hashlib

import numpy as np

WEIGHT_STD = 0.02

TENSOR_IDS = {
    "x": 1, "w": 2, "x_attn": 3, "w_o": 4, "x_ffn": 5, "w_down": 6,
    "residual": 7, "slots": 8, "logits": 9, "u": 10, "w_expert": 11,
    "partials": 12, "x_ffn_in": 13, "w_gate": 14, "w_up": 15, "x_qkv_in": 16, "w_qkv": 17,
}


def _key_ints(seed=0, workload=0, layer=0, tensor="x", rank=0):
    if isinstance(workload, str):
        workload = int.from_bytes(hashlib.sha256(workload.encode()).digest()[:4], "little")
    return [int(seed), int(workload), int(layer), TENSOR_IDS[tensor], int(rank)]


def rng(seed=0, workload=0, layer=0, tensor="x", rank=0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        _key_ints(seed, workload, layer, tensor, rank))))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7F800000) == 0x7F800000
    nan &= (u & 0x007FFFFF) != 0
    lower = u & 0xFFFF
    upper = u >> 16
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    out = (upper + up.astype(np.uint32)).astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, std=1.0, **key) -> np.ndarray:
    """N(0, std) samples as bf16 bit patterns (uint16)."""
    g = rng(**key)
    v = g.standard_normal(size=shape, dtype=np.float64) * std
    return f32_to_bf16_bits(v.astype(np.float32))


def normal_f32(shape, std=1.0, **key) -> np.ndarray:
    g = rng(**key)
    return (g.standard_normal(size=shape, dtype=np.float64) * std).astype(np.float32)


def _torch_seed(**key) -> int:
    h = hashlib.sha256(repr(_key_ints(**key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def device_normal(shape, std=1.0, dtype=None, device="cuda", **key):
    """N(0, std) on the device from torch's seeded generator, rounded to dtype.

    Used for benchmark-sized tensors (gigabytes), which numpy would take
    minutes to draw. float32 -> dtype rounding is torch's nearest-even.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(**key))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t if dtype is None else t.to(dtype)
