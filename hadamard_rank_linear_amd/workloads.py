"""Seeded synthetic layer inputs for the HLQ/HOT linear-layer backward.

This module only draws random numbers and rounds them to a storage dtype; it
holds none of the method's arithmetic, so both the GPU library's tests and the
CPU oracle may consume its buffers.

The five layer shapes stand in for the workloads the HOT summary page measures
("HOT: Hadamard-based Optimized Training", scime.ai summary, "Key results" and
the "Measured effects" table: ViT-B qkv and fc2 layers; Llama3-8B fine-tuning;
ResNet-50 at batch 256).  No dataset item is used: every tensor is drawn from
the distribution stated next to it.

Recipe: every tensor has its own numpy PCG64 stream seeded from
(seed, config index, tensor index); values are drawn in fp64, rounded to fp32
(round-to-nearest-even) and, for bf16 configs, rounded again to bf16
(round-to-nearest-even on the fp32 bit pattern).  bf16 tensors are returned as
uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = 0
BF16 = 1
PER_TOKEN = 0
PER_TENSOR = 1
SUM = 0
MEAN = 1


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    index: int
    name: str
    T: int
    I: int
    O: int
    dtype: int
    block: int
    rank: int
    gx_mode: int
    gw_mode: int
    reduction: int
    gy_dist: str
    x_dist: str
    w_dist: str

    def with_tokens(self, T: int) -> "LayerConfig":
        return dataclasses.replace(self, T=T)

    @property
    def Tl(self) -> int:
        return self.T * self.rank // self.block


LAYERS = [
    LayerConfig(0, "tiny", 256, 64, 64, F32, 16, 8, PER_TOKEN, PER_TOKEN, SUM,
                "normal(1)+1%x20", "normal(1)", "normal(0.02)"),
    LayerConfig(1, "vitb_qkv", 12608, 768, 2304, BF16, 16, 8, PER_TOKEN, PER_TENSOR, SUM,
                "normal(1e-3)+0.5%x50", "normal(1)", "normal(0.02)"),
    LayerConfig(2, "vitb_fc2", 12608, 3072, 768, BF16, 32, 8, PER_TOKEN, PER_TOKEN, SUM,
                "1e-3*student_t(4)", "gelu(normal(1))", "normal(0.02)"),
    LayerConfig(3, "llama3_8b_down", 4096, 14336, 4096, BF16, 64, 16, PER_TOKEN, PER_TOKEN, SUM,
                "1e-4*student_t(3)", "normal(1)*lognormal_channel(0,1)", "normal(0.01)"),
    LayerConfig(4, "resnet50_s3_conv", 50176, 2304, 256, BF16, 16, 4, PER_TENSOR, PER_TENSOR, SUM,
                "normal(1e-3)", "relu(normal(1))", "he_normal(2304)"),
]
BY_NAME = {c.name: c for c in LAYERS}


def _rng(seed: int, cfg: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, tensor])))


def _erf(x: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return erf(x)


def _draw(dist: str, shape, rng: np.random.Generator, cfg: LayerConfig) -> np.ndarray:
    T, I = shape if len(shape) == 2 else (None, None)
    if dist == "normal(1)":
        return rng.standard_normal(shape)
    if dist == "normal(0.02)":
        return 0.02 * rng.standard_normal(shape)
    if dist == "normal(0.01)":
        return 0.01 * rng.standard_normal(shape)
    if dist == "normal(1e-3)":
        return 1e-3 * rng.standard_normal(shape)
    if dist == "normal(1)+1%x20":
        v = rng.standard_normal(shape)
        v[rng.random(shape) < 0.01] *= 20.0
        return v
    if dist == "normal(1e-3)+0.5%x50":
        v = 1e-3 * rng.standard_normal(shape)
        v[rng.random(shape) < 0.005] *= 50.0
        return v
    if dist == "1e-3*student_t(4)":
        return 1e-3 * rng.standard_t(4, shape)
    if dist == "1e-4*student_t(3)":
        return 1e-4 * rng.standard_t(3, shape)
    if dist == "gelu(normal(1))":
        z = rng.standard_normal(shape)
        return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))
    if dist == "relu(normal(1))":
        return np.maximum(rng.standard_normal(shape), 0.0)
    if dist == "normal(1)*lognormal_channel(0,1)":
        c = rng.lognormal(0.0, 1.0, shape[1])
        return rng.standard_normal(shape) * c[None, :]
    if dist == "he_normal(2304)":
        return math.sqrt(2.0 / 2304.0) * rng.standard_normal(shape)
    if dist == "he_normal(fan_in)":   # fan-in = the feature count shape[1]
        return math.sqrt(2.0 / shape[1]) * rng.standard_normal(shape)
    raise ValueError(f"unknown distribution {dist!r}")


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _store(v64: np.ndarray, dtype: int) -> np.ndarray:
    v32 = v64.astype(np.float32)
    return v32 if dtype == F32 else f32_to_bf16_bits(v32)


def make_inputs(cfg: LayerConfig, seed: int = 0, plant_zero_rows: bool = False) -> dict:
    """Draw g_y [T x O], x [T x I] and w [O x I] for ``cfg``.

    Returns a dict with host arrays in the storage dtype (fp32, or uint16 bf16
    bit patterns).  ``plant_zero_rows`` zeroes token 0 of g_y and x and output
    row 0 of w, so that an all-zero scale group occurs (edge case).
    """
    gy = _draw(cfg.gy_dist, (cfg.T, cfg.O), _rng(seed, cfg.index, 0), cfg)
    x = _draw(cfg.x_dist, (cfg.T, cfg.I), _rng(seed, cfg.index, 1), cfg)
    w = _draw(cfg.w_dist, (cfg.O, cfg.I), _rng(seed, cfg.index, 2), cfg)
    if plant_zero_rows:
        gy[0, :] = 0.0
        x[0, :] = 0.0
        w[0, :] = 0.0
    return dict(gy=_store(gy, cfg.dtype), x=_store(x, cfg.dtype),
                w=_store(w, cfg.dtype), dtype=cfg.dtype)


# ---------------------------------------------------------------- convolutions

@dataclasses.dataclass(frozen=True)
class ConvConfig:
    """A 2-D convolution layer: NHWC input [N, H, W, C], OHWI weight
    [O, R, S, C], zero padding.  Tokens of its linear form are the output
    pixels (n, p, q); features are (r, s, c)."""
    index: int
    name: str
    N: int
    H: int
    W: int
    C: int
    O: int
    R: int
    S: int
    stride: int
    pad: int
    dtype: int
    block: int
    rank: int
    gx_mode: int
    gw_mode: int
    reduction: int
    gy_dist: str
    x_dist: str
    w_dist: str

    @property
    def P(self) -> int:
        return (self.H + 2 * self.pad - self.R) // self.stride + 1

    @property
    def Q(self) -> int:
        return (self.W + 2 * self.pad - self.S) // self.stride + 1

    @property
    def T(self) -> int:
        return self.N * self.P * self.Q

    @property
    def I(self) -> int:
        return self.R * self.S * self.C

    @property
    def Tl(self) -> int:
        return self.T * self.rank // self.block


CONV_LAYERS = [
    # ResNet-50 stage 3, 3x3 convolution at batch 256 (the im2col layer config
    # above, run as a convolution)
    ConvConfig(20, "resnet50_s3_conv3x3", 256, 14, 14, 256, 256, 3, 3, 1, 1, BF16, 16, 4,
               PER_TENSOR, PER_TENSOR, SUM, "normal(1e-3)", "relu(normal(1))", "he_normal(fan_in)"),
    # small strided, padded convolution
    ConvConfig(21, "small_stride2_pad1", 2, 15, 15, 16, 32, 3, 3, 2, 1, F32, 16, 8,
               PER_TENSOR, PER_TOKEN, SUM, "normal(1)", "relu(normal(1))", "he_normal(fan_in)"),
]
CONV_BY_NAME = {c.name: c for c in CONV_LAYERS}


def make_conv_inputs(cfg: ConvConfig, seed: int = 0) -> dict:
    """g_y [N*P*Q x O] (rows (n, p, q)), x [N*H*W x C] (rows (n, h, w)) and
    w [O x R*S*C] (OHWI) for ``cfg``, in the storage dtype."""
    gy = _draw(cfg.gy_dist, (cfg.T, cfg.O), _rng(seed, cfg.index, 0), cfg)
    x = _draw(cfg.x_dist, (cfg.N * cfg.H * cfg.W, cfg.C), _rng(seed, cfg.index, 1), cfg)
    w = _draw(cfg.w_dist, (cfg.O, cfg.I), _rng(seed, cfg.index, 2), cfg)
    return dict(gy=_store(gy, cfg.dtype), x=_store(x, cfg.dtype),
                w=_store(w, cfg.dtype), dtype=cfg.dtype)
