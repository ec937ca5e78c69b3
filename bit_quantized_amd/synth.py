"""Seeded synthetic inputs for the W4A8 linear layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no quantisation, no packing, no products).  Both the HIP
path and the CPU oracle receive the arrays made here, so neither side can feed
the other.

Shapes and distributions follow the layer the pages describe ("The 4-bit CPU
path", section "W4A8": GPTQ int4 weights with per-group metadata, int8
activations; section "Building a checkpoint": group size 128).  The per-group
asymmetric zero points are drawn as integers 0..15, the reading the same page
gives when it contrasts checkpoint zero points with the constant 8.

Draw order for one linear, from ``numpy.random.Generator(PCG64(seed))``:
  1. x ~ N(0, 1), float32, [M][K]
  2. outlier channels (bf16 activations only): round(0.005*K) distinct column
     indices, the same for every row, multiplied by 20
  3. x rounded to bfloat16 (round to nearest, ties to even) for bf16 inputs
  4. q ~ U{0..15}, uint8, [N][K]
  5. z ~ U{0..15}, uint8, [N][K/group]
  6. s = |N(0, 0.02)|, float32, [N][K/group]

For the W8A8 linear ("Serve a pre-quantized int8 weight-only DiT ...",
comment "Round two ...": int8 per-channel weights, int8 dynamic
activations) the weights are drawn instead as (``make_w8_linear``):
  4'. qw = clip(round(N(0, 32)), -127, 127), int8, [N][K]
  5'. one column per row, U{0..K-1}, set to +127 or -127 (U{+-1}): every
      channel reaches the full symmetric range, as a per-channel absmax grid does
  6'. sw = |N(0, 0.0005)|, float32, [N]
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

GROUP = 128

# 7B-decoder-shaped linears: hidden 3584, intermediate 18944, two 512-wide
# key/value heads, vocabulary 152064.
LAYER_LINEARS = (
    ("q", 3584, 3584),
    ("k", 3584, 512),
    ("v", 3584, 512),
    ("o", 3584, 3584),
    ("gate", 3584, 18944),
    ("up", 3584, 18944),
    ("down", 18944, 3584),
    ("head", 3584, 152064),
)


@dataclass(frozen=True)
class LinearSpec:
    name: str
    M: int
    K: int
    N: int
    seed: int
    act: str = "bf16_outliers"  # or "f32"
    group: int = GROUP


# Workloads used by tests and the benchmark.
TINY = LinearSpec("tiny", 4, 256, 256, seed=0, act="f32")
DECODE_UP = LinearSpec("decode_up", 1, 3584, 18944, seed=1)
SKINNY_DOWN_4 = LinearSpec("skinny_down_m4", 4, 18944, 3584, seed=2)
SKINNY_DOWN_16 = LinearSpec("skinny_down_m16", 16, 18944, 3584, seed=2)
# the same batches on the MLP up projection (the shape of the decode GEMV)
SKINNY_UP_4 = LinearSpec("skinny_up_m4", 4, 3584, 18944, seed=2)
SKINNY_UP_16 = LinearSpec("skinny_up_m16", 16, 3584, 18944, seed=2)
PREFILL_UP = LinearSpec("prefill_up", 2048, 3584, 18944, seed=3)


def layer_specs(M: int) -> list[LinearSpec]:
    """The seven layer linears plus the output head at M tokens."""
    return [LinearSpec(f"layer_{n}_m{M}", M, K, N, seed=4000 + i)
            for i, (n, K, N) in enumerate(LAYER_LINEARS)]


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs must be finite (the generator never makes anything else)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_activations(rng: np.random.Generator, M: int, K: int, act: str):
    x = rng.standard_normal((M, K), dtype=np.float32)
    if act == "f32":
        return x, None
    if act != "bf16_outliers":
        raise ValueError(f"unknown activation kind {act!r}")
    n_out = int(round(0.005 * K))
    cols = rng.choice(K, size=n_out, replace=False)
    x[:, cols] *= np.float32(20.0)
    return bf16_round_bits(x), np.sort(cols)


def draw_w8_weights(rng: np.random.Generator, N: int, K: int):
    qw = np.clip(np.rint(rng.normal(0.0, 32.0, size=(N, K))), -127, 127).astype(np.int8)
    cols = rng.integers(0, K, size=N)
    signs = rng.choice(np.array([-127, 127], dtype=np.int8), size=N)
    qw[np.arange(N), cols] = signs
    sw = np.abs(rng.normal(0.0, 0.0005, size=N)).astype(np.float32)
    return qw, sw


def make_w8_linear(spec: LinearSpec) -> dict:
    """One W8A8 linear's inputs: ``x`` (as make_linear), ``qw`` int8 [N][K]
    and ``sw`` float32 [N]."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    x, cols = draw_activations(rng, spec.M, spec.K, spec.act)
    qw, sw = draw_w8_weights(rng, spec.N, spec.K)
    return {"spec": spec, "x": x, "outlier_cols": cols, "qw": qw, "sw": sw}


def draw_weights(rng: np.random.Generator, N: int, K: int, group: int = GROUP):
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z = rng.integers(0, 16, size=(N, G), dtype=np.uint8)
    s = np.abs(rng.normal(0.0, 0.02, size=(N, G))).astype(np.float32)
    return q, z, s


def make_linear(spec: LinearSpec, with_weights: bool = True) -> dict:
    """Draw one linear's inputs.

    Returns ``x`` (float32 array for act="f32", else uint16 bf16 bit patterns),
    ``outlier_cols`` and, with weights, ``q``, ``z``, ``s``."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    x, cols = draw_activations(rng, spec.M, spec.K, spec.act)
    out = {"spec": spec, "x": x, "outlier_cols": cols}
    if with_weights:
        out["q"], out["z"], out["s"] = draw_weights(rng, spec.N, spec.K, spec.group)
    return out


def x_as_f32(lin: dict) -> np.ndarray:
    """Activations widened to float32 (exact for bf16)."""
    x = lin["x"]
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


def digest(lin: dict) -> str:
    """sha256 over the drawn arrays, recorded beside results."""
    h = hashlib.sha256()
    for k in ("x", "q", "z", "s"):
        if k in lin:
            h.update(np.ascontiguousarray(lin[k]).tobytes())
    return h.hexdigest()[:16]
