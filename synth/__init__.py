"""Seeded synthetic inputs for the ternary-weight linear layer.

This module only draws random numbers and rounds them into the storage types
the layer consumes: ternary codes as int8 values in {-1, 0, +1}, fp16 scale bit
patterns, bf16/fp16 activation bit patterns and raw random bytes.  None of the
layer's own arithmetic (packing, 2-bit decoding, scaling, accumulation) lives
here, so both the CPU oracle and the GPU path can consume these arrays without
sharing any of the method.

Workload recipe (shapes follow the models the pages describe; no weights or
datasets from those models are used):
  * codes: u ~ U[0,1) i.i.d. per weight; q = +1 if u < p_plus,
    -1 if u < p_plus + p_minus, else 0;
  * scales: U[0.005, 0.05] in fp64, rounded to fp16 (round-to-nearest-even);
  * activations: N(0, 1) in fp64, rounded to bf16 (round-to-nearest-even);
  * draw order within one case: codes, then scales, then activations.
Seeds: the tiny case uses ``default_rng(0)``; every other case uses
``default_rng(SeedSequence([config, shape_index, M]))``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Shape",
    "Config",
    "CONFIGS",
    "rng_for",
    "draw_codes",
    "draw_scales",
    "draw_x",
    "draw_bytes",
    "f64_to_bf16_bits",
    "f64_to_f16_bits",
    "Case",
    "make_case",
]


@dataclass(frozen=True)
class Shape:
    name: str
    N: int  # output channels (rows of the packed weight)
    K: int  # input features (reduction length)


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    shapes: tuple
    Ms: tuple
    group_size: int  # 128 or -1 (one scale per output channel)
    p_plus: float
    p_minus: float
    description: str = ""


_PROJ7B = (
    Shape("q", 4096, 4096),
    Shape("k", 512, 4096),
    Shape("v", 512, 4096),
    Shape("o", 4096, 4096),
    Shape("gate", 18944, 4096),
    Shape("up", 18944, 4096),
    Shape("down", 4096, 18944),
)

CONFIGS = {
    0: Config(0, "tiny-gemv", (Shape("w", 1024, 1024),), (1,), 128, 0.3, 0.3,
              "M=1, N=K=1024, group-128 scales"),
    1: Config(1, "embed-0.6b-mlp",
              (Shape("gate", 3072, 1024), Shape("up", 3072, 1024), Shape("down", 1024, 3072)),
              (1, 8, 64), 128, 0.3, 0.3,
              "0.6B-embedding-shaped MLP, group-128 scales"),
    2: Config(2, "7b-decode", _PROJ7B, (1, 8), -1, 0.3, 0.3,
              "7B-shaped attention+MLP projections, per-channel scales, decode"),
    3: Config(3, "7b-prefill", _PROJ7B, (2048,), -1, 0.3, 0.3,
              "7B-shaped projections at 2048 tokens, per-channel scales"),
    4: Config(4, "27b-sweep", (Shape("up", 25600, 5120), Shape("down", 5120, 25600)),
              (1, 4, 16, 64, 256), 128, 0.25, 0.25,
              "27B-class hidden 5120 / intermediate 25600, group-128 scales"),
}


def rng_for(config: int, shape_index: int = 0, M: int = 1) -> np.random.Generator:
    """Generator for one (config, shape, M) case."""
    if config == 0:
        return np.random.default_rng(0)
    return np.random.default_rng(np.random.SeedSequence([config, shape_index, M]))


_ROW_CHUNK_ELEMS = 1 << 24  # draw uniforms in row chunks to bound host memory


def draw_codes(rng: np.random.Generator, N: int, K: int,
               p_plus: float = 0.3, p_minus: float = 0.3) -> np.ndarray:
    """int8 [N, K] with P(+1)=p_plus, P(-1)=p_minus, P(0)=1-p_plus-p_minus."""
    out = np.empty((N, K), dtype=np.int8)
    rows = max(1, _ROW_CHUNK_ELEMS // max(K, 1))
    for r0 in range(0, N, rows):
        r1 = min(N, r0 + rows)
        u = rng.random((r1 - r0, K))
        blk = np.zeros((r1 - r0, K), dtype=np.int8)
        blk[u < p_plus] = 1
        blk[(u >= p_plus) & (u < p_plus + p_minus)] = -1
        out[r0:r1] = blk
    return out


def f64_to_f16_bits(a) -> np.ndarray:
    """fp64 -> IEEE binary16 bit patterns, round-to-nearest-even (numpy's cast)."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def f64_to_bf16_bits(a) -> np.ndarray:
    """fp64 -> bfloat16 bit patterns, round-to-nearest-even, for finite normal inputs.

    Rounds the significand to 8 bits directly from fp64 (no double rounding),
    then takes the upper half of the exactly representable fp32 value.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)                      # a = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(m * 256.0), e - 8)  # 8 significant bits, ties to even
    f32 = r.astype(np.float32)               # exact: 8-bit significand
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def draw_scales(rng: np.random.Generator, N: int, K: int, group_size: int,
                lo: float = 0.005, hi: float = 0.05) -> np.ndarray:
    """fp16 bit patterns, shape [N] (group_size == -1) or [N, K // group_size]."""
    shape = (N,) if group_size == -1 else (N, K // group_size)
    return f64_to_f16_bits(lo + (hi - lo) * rng.random(shape))


def draw_x(rng: np.random.Generator, M: int, K: int, dtype: str = "bf16") -> np.ndarray:
    """Activation bit patterns [M, K] (uint16), N(0,1) rounded to bf16 or fp16."""
    v = rng.standard_normal((M, K))
    if dtype == "bf16":
        return f64_to_bf16_bits(v)
    if dtype == "fp16":
        return f64_to_f16_bits(v)
    raise ValueError(f"unknown activation dtype {dtype!r}")


def draw_weights(rng: np.random.Generator, N: int, K: int, std: float = 0.02,
                 dtype: str = "bf16") -> np.ndarray:
    """Dense weight bit patterns [N, K] (uint16) for the quantizer: N(0, std^2)
    rounded to bf16 or fp16.  std = 0.02 is a common initialisation scale of
    linear layers; no trained weights are involved."""
    v = rng.standard_normal((N, K)) * std
    if dtype == "bf16":
        return f64_to_bf16_bits(v)
    if dtype == "fp16":
        return f64_to_f16_bits(v)
    raise ValueError(f"unknown weight dtype {dtype!r}")


def draw_bytes(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Uniform random bytes [N, K // 4]; these include the reserved 2-bit field."""
    return rng.integers(0, 256, size=(N, K // 4), dtype=np.uint8)


@dataclass
class Case:
    config: int
    shape: Shape
    M: int
    group_size: int
    codes: np.ndarray            # int8 [N, K]
    scale: np.ndarray            # uint16 fp16 bits
    x: np.ndarray                # uint16 bf16/fp16 bits [M, K]
    dtype: str = "bf16"
    meta: dict = field(default_factory=dict)


def make_case(config: int, shape_index: int, M: int, dtype: str = "bf16") -> Case:
    """Draw one case of a named workload (codes, scales, activations)."""
    cfg = CONFIGS[config]
    shp = cfg.shapes[shape_index]
    rng = rng_for(config, shape_index, M)
    codes = draw_codes(rng, shp.N, shp.K, cfg.p_plus, cfg.p_minus)
    scale = draw_scales(rng, shp.N, shp.K, cfg.group_size)
    x = draw_x(rng, M, shp.K, dtype)
    return Case(config, shp, M, cfg.group_size, codes, scale, x, dtype)
