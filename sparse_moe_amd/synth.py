"""Seeded synthetic inputs for the routed-MoE layer (Gemma 4 26B-A4B shape).

This module only draws random numbers and lays them out in the storage
formats the layer consumes: fp32 arrays, bf16 bit patterns, and ggml Q4_0
blocks of raw bytes (an fp16 scale followed by 16 bytes of packed 4-bit
codes).  It holds none of the layer's arithmetic: no dequantisation, no
products, no routing.  Both the CPU oracle's tests and the GPU path's tests
and benchmark draw their inputs from here, so the two sides see identical
bytes.

Shapes follow the model card "Gemma 4 26B-A4B it QAT Q4_0 with MTP assistant
and vision, NInfer v3 artifact", table "What is inside": 128 routed experts per
block, stored expert-major as Q4_0 with a [gate; up] parent of 2 x 704 rows and
a down matrix of 2,816 rows; the router, router scale and expert scales are
FP32.  Value distributions are the five synthetic workloads this project is
measured on (tiny layer, 1-token decode, 8-token decode, 4,096-token prefill,
30-layer stack).

Every tensor has its own random stream, keyed by (seed, tensor id), so adding
a tensor never shifts another one's values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# ---------------------------------------------------------------------------
# tensor ids (one random stream per id)
T_X = 0          # activations
T_WR = 1         # router weight [E, H]
T_GATE_UP = 2    # Q4_0 [E][2I rows][H/32 blocks]
T_DOWN = 3       # Q4_0 [E][H rows][I/32 blocks]
T_SCALE = 4      # per-expert output scale [E]
T_LOGITS = 5     # injected router logits [T, E]
T_RMS_W = 6      # RMSNorm weight [H]
T_ZIPF = 7       # random expert ranks for the Zipf prior [E]

Q4_0_BLOCK = 32          # weights per ggml Q4_0 block
Q4_0_BYTES = 18          # 2-byte fp16 scale + 16 bytes of nibbles


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id])))


def normal_f32(g: np.random.Generator, shape, mean: float, std: float) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std) + np.float32(mean)).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store fp32 samples as bf16 bit patterns (round to nearest even).

    Uses torch's CPU dtype conversion; this only fixes the input format."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def q4_0_random(g: np.random.Generator, lead: int, rows: int, cols: int,
                scale_std: float = 0.02) -> np.ndarray:
    """Random ggml Q4_0 matrix stack as raw bytes, shape [lead, rows, cols/32, 18].

    Scale: fp16 of |N(0, scale_std)| (little-endian, bytes 0-1 of a block);
    codes: uniform nibbles 0..15, i.e. 16 uniform random bytes (bytes 2-17)."""
    assert cols % Q4_0_BLOCK == 0
    nb = cols // Q4_0_BLOCK
    n = lead * rows * nb
    d = np.abs(g.standard_normal(n, dtype=np.float32) * np.float32(scale_std)).astype(np.float16)
    qs = np.frombuffer(g.bytes(n * 16), dtype=np.uint8).reshape(n, 16)
    out = np.empty((n, Q4_0_BYTES), dtype=np.uint8)
    out[:, 0:2] = d.view(np.uint8).reshape(n, 2)
    out[:, 2:] = qs
    return out.reshape(lead, rows, nb, Q4_0_BYTES)


# ---------------------------------------------------------------------------
@dataclass
class LayerSpec:
    name: str
    H: int
    E: int
    K: int
    I: int
    T: int
    act: str                  # "f32" or "bf16": dtype of x (and of the hidden h)
    router_std: float         # std of router weight entries
    seed: int
    zipf_s: Optional[float] = None   # additive log-prior on the router (stack workload)
    rms_eps: Optional[float] = None  # RMSNorm before the layer (stack workload)
    layers: int = 1


SPECS = {
    0: LayerSpec("tiny", H=256, E=8, K=2, I=64, T=4, act="f32", router_std=1.0 / 16, seed=0),
    1: LayerSpec("decode-1tok", H=2816, E=128, K=8, I=704, T=1, act="f32",
                 router_std=1.0 / math.sqrt(2816), seed=1),
    2: LayerSpec("decode-8tok", H=2816, E=128, K=8, I=704, T=8, act="bf16",
                 router_std=1.0 / math.sqrt(2816), seed=2),
    3: LayerSpec("prefill-4096", H=2816, E=128, K=8, I=704, T=4096, act="bf16",
                 router_std=1.0 / math.sqrt(2816), seed=3),
    4: LayerSpec("stack30-512", H=2816, E=128, K=8, I=704, T=512, act="bf16",
                 router_std=1.0 / math.sqrt(2816), seed=4, zipf_s=1.1, rms_eps=1e-6, layers=30),
}


@dataclass
class LayerInputs:
    spec: LayerSpec
    T: int
    x: np.ndarray                 # [T, H] float32, or uint16 bf16 bits
    w_router: np.ndarray          # [E, H] float32
    router_bias: Optional[np.ndarray]   # [E] float32 or None
    w_gate_up: np.ndarray         # uint8 [E, 2I, H/32, 18]
    w_down: np.ndarray            # uint8 [E, H, I/32, 18]
    expert_scale: np.ndarray      # [E] float32
    rms_w: Optional[np.ndarray] = None  # [H] float32 (stack only)
    extra: dict = field(default_factory=dict)


def activations(spec: LayerSpec, T: int, seed: int) -> np.ndarray:
    x = normal_f32(rng(seed, T_X), (T, spec.H), 0.0, 1.0)
    return x if spec.act == "f32" else f32_to_bf16_bits(x)


def zipf_bias(g: np.random.Generator, E: int, s: float) -> np.ndarray:
    """Additive router prior: bias[e] = -s * ln(rank_e) with ranks a random
    permutation of 1..E, so that the prior weight of an expert is rank^-s."""
    ranks = g.permutation(E) + 1
    return (-s * np.log(ranks.astype(np.float64))).astype(np.float32)


def make_layer(spec: LayerSpec, seed: Optional[int] = None, T: Optional[int] = None,
               with_x: bool = True) -> LayerInputs:
    seed = spec.seed if seed is None else seed
    T = spec.T if T is None else T
    H, E, I = spec.H, spec.E, spec.I
    x = activations(spec, T, seed) if with_x else None
    w_r = normal_f32(rng(seed, T_WR), (E, H), 0.0, spec.router_std)
    gu = q4_0_random(rng(seed, T_GATE_UP), E, 2 * I, H)
    dn = q4_0_random(rng(seed, T_DOWN), E, H, I)
    sc = normal_f32(rng(seed, T_SCALE), (E,), 1.0, 0.1)
    bias = zipf_bias(rng(seed, T_ZIPF), E, spec.zipf_s) if spec.zipf_s else None
    rms_w = normal_f32(rng(seed, T_RMS_W), (H,), 1.0, 0.05) if spec.rms_eps else None
    return LayerInputs(spec, T, x, w_r, bias, gu, dn, sc, rms_w)


def stack_layer_seed(layer: int) -> int:
    """Independent seed of layer l of the 30-layer stack."""
    return 4000 + layer


def uniform_logits(T: int, E: int, seed: int) -> np.ndarray:
    """Injected router logits ~ U(0, 1) (the router bypass mode)."""
    return rng(seed, T_LOGITS).random((T, E), dtype=np.float32)
