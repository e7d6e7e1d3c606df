"""Seeded synthetic inputs for the nested W4/W8 linear.

This module draws random tensors and nothing else: it holds none of the
method's arithmetic (no unpacking, dequantisation, quantisation or products),
so both the HIP path and the CPU oracle can take their inputs from it.

Recipe (the shapes are Llama-3-8B's decoder linears, the base model named on
the BitNest-Llama-3-8B model card; the distributions stand in for the real
weight package, which is not available):

* plane bytes: each byte holds two independent nibbles drawn from the same
  distribution, so which nibble is which column does not matter to the draw.
  hi nibbles: clamp(round(N(0, 2.5)) + 8, 0, 15); lo nibbles: uniform 0..15.
* scales: fp16(lognormal(log 0.01, 0.3)), one per row and 128 columns.
* activations: fp32 N(0, 1); in the layer workloads round(0.005 K) channels,
  the same for every token of a call, are multiplied by 20 (outliers).

Every tensor has its own seed, derived from (seed, layer, linear, tensor,
decoding step) by
numpy's SeedSequence, and is drawn with torch's generator on the device the
tensor is made on (CPU and GPU generators give different, equally seeded,
streams).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

GROUP = 128

# Llama-3-8B decoder linears, with q/k/v and gate/up fused along N.
# (name, N, K, act_group): o_proj takes per-128-group activation scales.
LLAMA3_8B_LINEARS = (
    ("qkv", 6144, 4096, 0),
    ("o_proj", 4096, 4096, 128),
    ("gate_up", 28672, 4096, 0),
    ("down", 4096, 14336, 0),
)
LLAMA3_8B_LAYERS = 32

_TENSOR_IDS = {"hi": 0, "lo": 1, "scale": 2, "x": 3, "outliers": 4}


def derive_seed(seed: int, layer: int, linear: int, tensor: str, step: int = 0) -> int:
    ss = np.random.SeedSequence([int(seed), int(layer), int(linear), _TENSOR_IDS[tensor], int(step)])
    return int(ss.generate_state(1, np.uint64)[0] >> np.uint64(1))


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _hi_nibbles(shape, g, device):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * 2.5
    return (torch.round(t) + 8).clamp_(0, 15).to(torch.uint8)


def _lo_nibbles(shape, g, device):
    return torch.randint(0, 16, shape, generator=g, device=device, dtype=torch.uint8)


def _two_nibble_bytes(draw, N: int, nbytes: int, g, device, row_block: int = 4096) -> torch.Tensor:
    out = torch.empty((N, nbytes), dtype=torch.uint8, device=device)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        a = draw((r1 - r0, nbytes), g, device)
        b = draw((r1 - r0, nbytes), g, device)
        out[r0:r1] = a | (b << 4)
    return out


@dataclass
class LinearWeights:
    hi: torch.Tensor       # uint8 [N, K/2]
    lo: torch.Tensor       # uint8 [N, K/2] (None if not drawn)
    scale: torch.Tensor    # int16 [N, K/128], fp16 bit patterns
    N: int
    K: int

    def to(self, device):
        return LinearWeights(self.hi.to(device), None if self.lo is None else self.lo.to(device),
                             self.scale.to(device), self.N, self.K)

    def numpy(self):
        """(hi, lo, scale) as numpy arrays: uint8, uint8 (or None), uint16."""
        hi = self.hi.cpu().numpy()
        lo = None if self.lo is None else self.lo.cpu().numpy()
        sc = self.scale.cpu().numpy().view(np.uint16)
        return hi, lo, sc


def make_weights(N: int, K: int, seed: int = 0, layer: int = 0, linear: int = 0,
                 with_lo: bool = True, device="cpu") -> LinearWeights:
    if K % GROUP:
        raise ValueError("K must be a multiple of %d" % GROUP)
    hi = _two_nibble_bytes(_hi_nibbles, N, K // 2,
                           _gen(device, derive_seed(seed, layer, linear, "hi")), device)
    lo = None
    if with_lo:
        lo = _two_nibble_bytes(_lo_nibbles, N, K // 2,
                               _gen(device, derive_seed(seed, layer, linear, "lo")), device)
    g = _gen(device, derive_seed(seed, layer, linear, "scale"))
    z = torch.randn((N, K // GROUP), generator=g, device=device, dtype=torch.float32)
    scale = torch.exp(math.log(0.01) + 0.3 * z).to(torch.float16).view(torch.int16)
    return LinearWeights(hi, lo, scale, N, K)


def n_outliers(K: int) -> int:
    return int(round(0.005 * K))


def make_activations(M: int, K: int, seed: int = 0, layer: int = 0, linear: int = 0,
                     outliers: bool = True, device="cpu", step: int = 0) -> torch.Tensor:
    """fp32 [M, K]; `step` tells apart the inputs of successive decoding steps."""
    g = _gen(device, derive_seed(seed, layer, linear, "x", step))
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    if outliers:
        go = _gen("cpu", derive_seed(seed, layer, linear, "outliers", step))
        idx = torch.randperm(K, generator=go)[: n_outliers(K)].to(device)
        x[:, idx] *= 20.0
    return x


def config0(seed: int = 0, device="cpu"):
    """Single linear N=256, K=512, M=1, no outliers."""
    w = make_weights(256, 512, seed=seed, layer=0, linear=0, device=device)
    x = make_activations(1, 512, seed=seed, layer=0, linear=0, outliers=False, device=device)
    return w, x
