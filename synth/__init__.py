"""Seeded synthetic inputs for the LittleBit layer forward.

This module only draws random numbers and rounds them to the storage types the
layer consumes (fp16 scales, bf16 activations). It holds none of the layer's
arithmetic: no rank rule, no sign packing, no contraction. Both the CPU oracle
and the HIP path read their inputs from here, so a test compares the two on the
same data.

Workload recipe (the shapes of the Llama2 and Qwen3 linears named in the
configuration table below; the factor and scale distributions follow the
description of the layer on the sesamedisk page, "How low-rank binarization
works": signed latent factors, three FP16 scale vectors h, g, l):

* latent factors U [d_out][r_p] and V [d_in][r_p] are fp32 N(0, 1); only their
  signs matter to the layer;
* scales h [d_out], g [d_in], l [r_p] are U(0.5, 1.5) rounded to fp16;
* activations x [T][d_in] are fp32 N(0, 1), rounded to bf16 (round to nearest
  even) for the bf16 workloads;
* draw order per linear: for each path p = 0, 1: U, V, h, g, l, from
  numpy Generator(PCG64(seed)); activations use their own seed.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# storage-type rounding (input preparation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)  # keep NaN quiet
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f16_bits(a: np.ndarray) -> np.ndarray:
    """fp32/fp64 values -> fp16 (numpy's round to nearest even) -> uint16 bits."""
    return np.ascontiguousarray(np.asarray(a).astype(np.float16)).view(np.uint16)


# ----------------------------------------------------------------------------
# one linear layer
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class LayerInputs:
    """Float factors and fp16 scales of one linear, all paths stacked path-major."""
    d_in: int
    d_out: int
    r_path: int
    paths: int
    U: np.ndarray   # float32 [P][d_out][r_path]
    V: np.ndarray   # float32 [P][d_in][r_path]
    h: np.ndarray   # uint16 fp16 bits [P][d_out]
    g: np.ndarray   # uint16 fp16 bits [P][d_in]
    l: np.ndarray   # uint16 fp16 bits [P][r_path]


def layer_inputs(seed: int, d_in: int, d_out: int, r_path: int, paths: int,
                 scale_lo: float = 0.5, scale_hi: float = 1.5) -> LayerInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    U = np.empty((paths, d_out, r_path), np.float32)
    V = np.empty((paths, d_in, r_path), np.float32)
    h = np.empty((paths, d_out), np.uint16)
    g = np.empty((paths, d_in), np.uint16)
    l = np.empty((paths, r_path), np.uint16)
    for p in range(paths):
        U[p] = rng.standard_normal((d_out, r_path), dtype=np.float32)
        V[p] = rng.standard_normal((d_in, r_path), dtype=np.float32)
        h[p] = f16_bits(rng.uniform(scale_lo, scale_hi, d_out))
        g[p] = f16_bits(rng.uniform(scale_lo, scale_hi, d_in))
        l[p] = f16_bits(rng.uniform(scale_lo, scale_hi, r_path))
    return LayerInputs(d_in, d_out, r_path, paths, U, V, h, g, l)


def unit_gain_l(d_in: int, r_path: int, paths: int) -> float:
    """Factor on the l draw that gives a linear an output RMS near its input's
    (signs are +-1, so each contraction grows a norm by about the square root
    of its length).  Used for layers chained one into the next, whose
    activations would otherwise grow layer by layer."""
    return 1.0 / float(np.sqrt(d_in * r_path * paths))


def dense_weight(seed: int, d_out: int, d_in: int, decay: float = 0.6, rms: float = 0.02) -> np.ndarray:
    """A dense fp32 weight [d_out][d_in] to initialise a layer from: random
    orthonormal singular vectors (QR of Gaussian draws) and singular values
    (1 + i)^-decay, scaled to the given entry RMS (a decaying spectrum, as
    trained weights have; distinct values, so the top singular vectors are
    well defined)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = min(d_out, d_in)
    a, _ = np.linalg.qr(rng.standard_normal((d_out, k)))
    b, _ = np.linalg.qr(rng.standard_normal((d_in, k)))
    s = (1.0 + np.arange(k)) ** -decay
    W = (a * s[None, :]) @ b.T
    W *= rms / np.sqrt(np.mean(W * W))
    return W.astype(np.float32)


def activations(seed: int, T: int, d: int, dtype: str) -> np.ndarray:
    """x [T][d]: float32 array for dtype 'f32', uint16 bf16 bits for 'bf16'."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((T, d), dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def activation_seed(seed: int) -> int:
    """Activations draw from their own stream, offset from the layer seed."""
    return 1_000_003 + seed


# ----------------------------------------------------------------------------
# the workload table (shapes and budgets; ranks are derived by the method)
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class LinearShape:
    name: str
    d_in: int
    d_out: int


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    title: str
    linears: Tuple[LinearShape, ...]
    b_num: int            # bits-per-weight budget b = b_num / b_den
    b_den: int
    residual: bool
    tokens: Tuple[int, ...]
    dtype: str            # activation dtype in and out: 'f32' or 'bf16'
    layers: int           # stack depth (1 = single layer)
    mlp: bool = False     # gate/up/down form one SwiGLU block
    heads: Tuple[int, int] = (0, 0)   # attention heads and kv heads of the model (decoder layers)


def _llama_like(d: int, ff: int, kv: int) -> Tuple[LinearShape, ...]:
    return (LinearShape("q", d, d), LinearShape("k", d, kv), LinearShape("v", d, kv),
            LinearShape("o", d, d), LinearShape("gate", d, ff), LinearShape("up", d, ff),
            LinearShape("down", ff, d))


WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", "single LittleBit linear 1024x1024, 1.0 bpw, no residual",
                   (LinearShape("linear", 1024, 1024),), 1, 1, False, (1, 8), "f32", 1),
    "c2": Workload("c2", "Qwen3-0.6B-shaped SwiGLU MLP 1024->3072->1024, 0.55 bpw + residual",
                   (LinearShape("gate", 1024, 3072), LinearShape("up", 1024, 3072),
                    LinearShape("down", 3072, 1024)), 55, 100, True, (1, 16), "bf16", 1, mlp=True),
    "c3": Workload("c3", "Llama2-7B-shaped decoder-layer linears, 1.0 bpw + residual, 32-layer stack",
                   _llama_like(4096, 11008, 4096), 1, 1, True, (1, 4, 32), "bf16", 32,
                   heads=(32, 32)),
    "c4": Workload("c4", "Qwen3-14B-shaped layer linears, 0.55 bpw + residual, 40-layer stack",
                   _llama_like(5120, 17408, 1024), 55, 100, True, (1, 2048), "bf16", 40,
                   heads=(40, 8)),
    "c5": Workload("c5", "Llama2-70B-shaped layer linears, 0.1 bpw + residual, 80-layer stack",
                   _llama_like(8192, 28672, 1024), 1, 10, True, (1, 2048), "bf16", 80,
                   heads=(64, 8)),
}


def layer_seed(layer: int, linear_index: int) -> int:
    """Seed of linear `linear_index` in stack layer `layer` (layer l uses seed l)."""
    return layer * 16 + linear_index


# ----------------------------------------------------------------------------
# device-side generation for large layer stacks
# ----------------------------------------------------------------------------

def device_layer(seed: int, d_in: int, d_out: int, r_path: int, paths: int, device="cuda"):
    """The same distributions drawn on the GPU with torch's seeded generator
    (for layer stacks too large to draw on the host quickly).  Returns float32
    U [P][d_out][r_path], V [P][d_in][r_path] and float16 h, g, l, all on
    `device`.  Draw order: U, V, h, g, l."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    U = torch.randn((paths, d_out, r_path), generator=gen, device=device, dtype=torch.float32)
    V = torch.randn((paths, d_in, r_path), generator=gen, device=device, dtype=torch.float32)
    unif = lambda shape: (torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
                          + 0.5).to(torch.float16)
    h = unif((paths, d_out))
    g = unif((paths, d_in))
    l = unif((paths, r_path))
    return U, V, h, g, l


def device_activations(seed: int, T: int, d: int, dtype: str, device="cuda"):
    """x [T][d] ~ N(0, 1) drawn on the GPU, as float32 or bfloat16 (RNE)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn((T, d), generator=gen, device=device, dtype=torch.float32)
    return x if dtype == "f32" else x.to(torch.bfloat16)
